/*
 * dsa.h -- C ABI of the DeepSeek Sparse Attention (DSA) forward path on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (page "DeepSeek-V3.2: sparse attention, scaled RL and synthetic
 * agent environments", Sec. 1.1, Eq. (1) and (2); Sec. 5.1; Sec. 5.2 Eq. (19)):
 *
 *   I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s])            lightning indexer
 *   S_t    = the k positions s <= t with the largest I[t,s] token selection
 *   u_t    = softmax-weighted sum over S_t of the latent   sparse MLA (MQA mode)
 *            rows c_s, every row shared by all query heads
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor pointers are DEVICE pointers, dense and row-major, owned by
 *   the caller.  The library allocates no memory; the calls that need
 *   scratch space take a caller-owned workspace (size from *_workspace_size).
 * - Outputs must not alias inputs or each other.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *   work is enqueued asynchronously on it; a call returns without waiting.
 * - The return value is a dsa_status.  Host-side validation happens before
 *   any HIP call: on a validation failure nothing is launched and outputs are
 *   untouched.  A failed launch returns DSA_ERR_HIP.  Faults inside kernels
 *   surface at the caller's next synchronisation.
 * - dsa_last_error() returns a thread-local description of the last failure.
 * - Element types: "e4m3" is an OCP FP8 E4M3FN byte; "bf16" is a bfloat16
 *   bit pattern in a uint16_t; scales and scores are IEEE float32.
 *
 * Positions: query row i (0 <= i < n_q) of a sequence sits at absolute
 * position p = q_pos0 + i and sees the n_p = min(p + 1, n_kv) cache entries
 * s = 0 .. n_p - 1 (s <= p: a token sees itself).  It selects
 * m_p = min(topk, n_p) of them (short rows select everything, Sec. 5.1).
 * Requires 0 <= q_pos0 and q_pos0 + n_q <= n_kv.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dsa_dims {
  int32_t batch;     /* B: independent sequences                                  */
  int32_t n_q;       /* T: query rows per sequence                                */
  int32_t n_kv;      /* S: cached tokens per sequence                             */
  int32_t q_pos0;    /* absolute position of query row 0 (prefill 0, decode S-1)  */
  int32_t idx_heads; /* H_I: indexer heads, 1..64                                 */
  int32_t idx_dim;   /* d_I: indexer head dim, multiple of 16, 16..128            */
  int32_t heads;     /* H: attention query heads, 1..128                          */
  int32_t dim_qk;    /* Dk: latent row width (keys), multiple of 16, <= 576       */
  int32_t dim_v;     /* Dv: value width = first Dv dims of a row, mult. of 32, <= 512, <= Dk */
  int32_t topk;      /* k: selected entries per query, 1..2048                    */
} dsa_dims;

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* null pointer, inconsistent dims, bad scale, ld too small */
  DSA_ERR_UNSUPPORTED = 2, /* dims outside what the kernels are built for          */
  DSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required            */
  DSA_ERR_HIP = 4          /* a HIP launch or runtime call failed                   */
} dsa_status;

/*
 * Lightning indexer scores (Eq. (1), Sec. 1.1).  FP8 inputs with one fp32
 * scale per token: the indexer query of head j of row i is
 * q_scale[b,i] * e4m3(q_idx[b,i,j,:]) and the key of entry s is
 * k_scale[b,s] * e4m3(k_idx[b,s,:]).
 *
 *   q_idx   [B, T, H_I, d_I] e4m3     q_scale [B, T] f32 (> 0, finite)
 *   w_idx   [B, T, H_I]      bf16     head weights w[t,j]
 *   k_idx   [B, S, d_I]      e4m3     k_scale [B, S] f32 (> 0, finite)
 *   scores  [B, T, ld]       f32      out: scores[b,i,s] = I[p,s] for s < n_p;
 *                                      entries s >= n_p are not written.
 *   ld >= n_kv (row stride of scores, in elements).
 * Products are exact FP8 x FP8 and summed in fp32; the ReLU, head weighting
 * and head sum are done in fp32.  The kernels do not check the scale values
 * (a NaN scale gives NaN scores, which top-k ranks last); dsa_validate counts
 * non-finite or non-positive scales on request.
 */
int dsa_indexer_scores(const dsa_dims* dims, const uint8_t* q_idx, const float* q_scale,
                       const uint16_t* w_idx, const uint8_t* k_idx, const float* k_scale,
                       float* scores, int64_t ld, void* stream);

/*
 * Top-k selection (S_t, Sec. 1.1 and Eq. (4); short rows Sec. 5.1; ties
 * Sec. 5.2 around Eq. (18)).  For every row, among scores[b,i,0:n_p] choose
 * the m_p largest; equal scores go to the lower index; NaN ranks below every
 * number; -0.0 equals +0.0.
 *
 *   scores [B, T, ld] f32 (only s < n_p is read), ld >= n_kv
 *   idx    [B, T, topk] int32 out: the chosen s in ascending order, then -1
 *          up to topk entries.
 * Supports n_kv <= 262144.
 */
int dsa_topk(const dsa_dims* dims, const float* scores, int64_t ld, int32_t* idx, void* stream);

/*
 * dsa_topk with a caller workspace of dsa_topk_workspace_size(dims) bytes
 * (256-byte aligned; the size is 0, and ws may be NULL, when no split
 * applies).  With a workspace, few long rows (at most 128 rows of at least
 * 16384 keys, e.g. a decode step) spread each row's candidate collection
 * over several workgroups, as dsa_forward does for its chunks.  The
 * selection is the same, bit for bit, as dsa_topk's.
 */
size_t dsa_topk_workspace_size(const dsa_dims* dims);
int dsa_topk_ws(const dsa_dims* dims, const float* scores, int64_t ld, int32_t* idx, void* ws, size_t ws_bytes,
                void* stream);

/*
 * Sparse MLA attention in MQA mode (Eq. (2), Sec. 1.1; renormalised softmax
 * over the selected set, Eq. (19), Sec. 5.2).  For every head h of row i:
 *   z_s   = sm_scale * sum_{d<Dk} q[b,i,h,d] * kv[b,s,d]       s in the row's set
 *   out   = sum_s softmax(z)_s * kv[b,s,0:Dv]
 *   lse   = max_s z_s + log(sum_s exp(z_s - max_s z_s))
 * The set of row i is {idx[b,i,j] : j < topk, 0 <= idx[b,i,j] < n_kv};
 * other entries (e.g. -1 padding) are skipped.  A row with an empty set
 * gets out = 0 and lse = -inf.
 *
 *   q    [B, T, H, Dk]  bf16       kv  [B, S, Dk] bf16
 *   idx  [B, T, topk]   int32      out [B, T, H, Dv] bf16
 *   lse  [B, T, H]      f32 or NULL
 *   ws   workspace of at least dsa_attn_workspace_size(dims) bytes (may be
 *        NULL when that size is 0).
 * QK^T and PV run on bf16 MFMA with fp32 accumulation; softmax is fp32.
 * One sequence's latent cache must be below 4 GiB (n_kv * Dk * 2 bytes <
 * 2^32, i.e. n_kv < 3,728,270 at Dk = 576): rows are addressed by 32-bit
 * offsets from the sequence's base.  Larger caches return
 * DSA_ERR_UNSUPPORTED.
 */
size_t dsa_attn_workspace_size(const dsa_dims* dims);
int dsa_sparse_mla_attn(const dsa_dims* dims, const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                        float sm_scale, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * dsa_sparse_mla_attn without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The split partials that
 * dsa_attn_workspace_size(dims) bytes would hold live in a static device
 * array of the library instead: 40 MiB per GPU, held from the first use of
 * the library on that GPU until the process ends (the 64-row decode step at
 * 128 heads x 512 dims needs 33.7 MB).  Dims needing more return
 * DSA_ERR_UNSUPPORTED before any launch.  The call allocates nothing; its
 * results equal dsa_sparse_mla_attn's bit for bit.  Every call on one GPU
 * shares that array: calls that may overlap in time on one GPU (on
 * different streams without ordering between them) race and must not be
 * issued; calls ordered on one stream are safe.
 */
int dsa_sparse_mla_attn_noalloc(const dsa_dims* dims, const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                                float sm_scale, uint16_t* out, float* lse, void* stream);

/*
 * The whole forward path: indexer -> top-k -> sparse MLA, processed in
 * chunks of query rows so that each chunk's scores stay in a workspace
 * slice (the workspace also holds the selection, the attention's split
 * partials and, for a few long rows, the top-k's per-part candidate lists).
 * Inputs and outputs are those of the three calls above.
 *   idx_out  [B, T, topk] int32 or NULL: if given, receives the selection.
 * The result equals, bit for bit, running dsa_indexer_scores, dsa_topk and
 * dsa_sparse_mla_attn one after the other.
 * ws must hold dsa_forward_workspace_size(dims) bytes (256-byte aligned).
 * Every launch goes to `stream`, chunk after chunk; the call needs no host
 * synchronisation, allocates nothing and may be captured in a HIP graph.
 */
size_t dsa_forward_workspace_size(const dsa_dims* dims);

/*
 * How dsa_forward (and dsa_forward_paged / dsa_forward_kl) splits its work
 * for these dims, for callers that time or reproduce its stages:
 *   chunk_rows      query rows per chunk (the last chunk may be shorter);
 *                   a chunk's scores are [B, chunk_rows, n_kv] f32
 *   topk_parts      top-k workgroups per row (1; or the parts of the split
 *                   selection that dsa_topk_ws also uses)
 *   attn_splits     attention workgroups per row (1; or split-k partials
 *                   merged by a log-sum-exp combine)
 *   workspace_bytes dsa_forward_workspace_size(dims)
 */
typedef struct dsa_forward_plan {
  int64_t chunk_rows;
  int32_t topk_parts;
  int32_t attn_splits;
  size_t workspace_bytes;
} dsa_forward_plan;
int dsa_forward_plan_of(const dsa_dims* dims, dsa_forward_plan* plan);

int dsa_forward(const dsa_dims* dims, const uint8_t* q_idx, const float* q_scale, const uint16_t* w_idx,
                const uint8_t* k_idx, const float* k_scale, const uint16_t* q, const uint16_t* kv,
                float sm_scale, uint16_t* out, float* lse, int32_t* idx_out, void* ws, size_t ws_bytes,
                void* stream);

/*
 * Per-token FP8 quantisation: the step that produces the FP8 indexer inputs
 * (the indexer runs in FP8, Sec. 1.1).  Format: OCP E4M3FN with one fp32
 * scale per token.  For each token t (token_len values x):
 *   scales[t]   = amax_t / 448, a correctly rounded fp32 division
 *                 (1.0 when amax_t == 0)
 *   codes[t, j] = e4m3(x[t, j] / scales[t]), the division correctly rounded
 *                 in fp32 and the conversion rounding to nearest, ties to
 *                 even, saturating at +-448 (a -0.0 quotient gives 0x80)
 *
 *   x       [n_tokens, token_len]  f32 (x_dtype 0) or bf16 (x_dtype 1),
 *           finite values (non-finite input gives unspecified codes)
 *   codes   [n_tokens, token_len]  e4m3 out
 *   scales  [n_tokens]             f32 out
 * token_len: a multiple of 4 in [4, 16384].  x must be 16-byte aligned for
 * f32 and 8-byte aligned for bf16; codes 4-byte aligned.
 */
int dsa_quantize_e4m3(const void* x, int x_dtype, int64_t n_tokens, int32_t token_len, uint8_t* codes,
                      float* scales, void* stream);

/*
 * Decode cache append: the n_q new tokens of every sequence, at positions
 * q_pos0 .. q_pos0 + n_q - 1, are written into the caches the calls above
 * read (a new token is in the cache before it attends, so with
 * q_pos0 = n_kv - 1 the decode query sees itself):
 *   k_new   [B, n_q, d_I]  f32 or bf16 (k_dtype 0 / 1), quantised exactly as
 *           by dsa_quantize_e4m3 into k_idx [B, n_kv, d_I] and
 *           k_scale [B, n_kv]
 *   kv_new  [B, n_q, Dk]   bf16, copied into kv [B, n_kv, Dk]
 * Other cache rows are untouched.  kv_new and kv may both be NULL to skip
 * the latent copy.  Uses batch, n_q, n_kv, q_pos0, idx_dim and dim_qk of
 * dims (dim_qk: a multiple of 8).
 */
int dsa_cache_append(const dsa_dims* dims, const void* k_new, int k_dtype, const uint16_t* kv_new,
                     uint8_t* k_idx, float* k_scale, uint16_t* kv, void* stream);

/*
 * Paged, variable-length caches (the analysis page, Sec. 5.1: the sequences
 * of one batch have their own context lengths, which limit each row to
 * min(k, t) candidates, and a row's selected entries are gathered from cache
 * pages, few and contiguous or many and scattered).
 *
 * Pools of num_pages pages of page_size tokens replace the [B, n_kv, ...]
 * caches:
 *   k_idx   [num_pages * page_size, d_I]  e4m3
 *   k_scale [num_pages * page_size]       f32
 *   kv      [num_pages * page_size, Dk]   bf16
 * Token s of sequence b is pool row
 *   page_table[b * max_pages + s / page_size] * page_size + s % page_size.
 * With page_table NULL the caches keep the dense [B, n_kv, ...] layout of the
 * calls above and only the lengths vary.
 *
 * Sequence b holds seq_lens[b] tokens; its n_q query rows are its last n_q
 * tokens, row i at position seq_lens[b] - n_q + i (a decode step: n_q = 1,
 * p = seq_lens[b] - 1, the new token sees itself), so row i has
 * seq_lens[b] - n_q + i + 1 candidates.  dims->n_kv bounds the lengths (and
 * is the scores row length); dims->q_pos0 is not used.  Query-side tensors
 * (q_idx, q_scale, w_idx, q, out, lse, scores, idx) keep their [B, n_q, ...]
 * layouts, and idx holds token indices s, not pool rows.
 *
 * seq_lens and page_table are device arrays whose values the host does not
 * read: a length outside [n_q, n_kv] is clamped into it and a page entry
 * outside [0, num_pages) is clamped into it (the results are then wrong, but
 * no access leaves the buffers).  Workspace sizes are those of the dense
 * calls (dsa_attn_workspace_size, dsa_forward_workspace_size).
 */
typedef struct {
  const int32_t* seq_lens;    /* device [B], required                                 */
  const int32_t* page_table;  /* device [B, max_pages], or NULL for dense caches      */
  int32_t page_size;          /* tokens per page, a positive multiple of 64            */
  int32_t max_pages;          /* row stride of page_table; max_pages * page_size >= n_kv */
  int32_t num_pages;          /* pages per pool; num_pages * page_size < 2^31          */
} dsa_paged_kv;

/* dsa_indexer_scores over a paged / variable-length key cache.  Row i of
 * sequence b is written for s < seq_lens[b] - n_q + i + 1. */
int dsa_indexer_scores_paged(const dsa_dims* dims, const dsa_paged_kv* layout, const uint8_t* q_idx,
                             const float* q_scale, const uint16_t* w_idx, const uint8_t* k_idx,
                             const float* k_scale, float* scores, int64_t ld, void* stream);
/* dsa_topk with per-sequence lengths (only layout->seq_lens is used). */
int dsa_topk_paged(const dsa_dims* dims, const dsa_paged_kv* layout, const float* scores, int64_t ld,
                   int32_t* idx, void* stream);
/* dsa_sparse_mla_attn over a paged / variable-length latent cache; entries
 * of idx outside [0, seq_lens[b]) are skipped.  A pool may exceed 4 GiB. */
int dsa_sparse_mla_attn_paged(const dsa_dims* dims, const dsa_paged_kv* layout, const uint16_t* q,
                              const uint16_t* kv, const int32_t* idx, float sm_scale, uint16_t* out, float* lse,
                              void* ws, size_t ws_bytes, void* stream);
/* dsa_forward over paged / variable-length caches: equal, bit for bit, to
 * the three paged calls one after the other. */
int dsa_forward_paged(const dsa_dims* dims, const dsa_paged_kv* layout, const uint8_t* q_idx,
                      const float* q_scale, const uint16_t* w_idx, const uint8_t* k_idx, const float* k_scale,
                      const uint16_t* q, const uint16_t* kv, float sm_scale, uint16_t* out, float* lse,
                      int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Locality counters of the selections (Sec. 5.1 of the analysis page: the
 * distinct pages, the contiguous runs and the hits per page of each row).
 * For every row of idx [B, n_q, topk] (ascending token indices as dsa_topk
 * writes them; entries < 0 skipped):
 *   stats[b, i, 0] = number of distinct pages s / page_size
 *   stats[b, i, 1] = number of maximal runs of consecutive indices
 *   stats[b, i, 2] = largest number of selected tokens on one page
 * stats is [B, n_q, 3] int32; an empty row gives 0 0 0.  Uses batch, n_q and
 * topk of dims; page_size >= 1.
 */
int dsa_gather_stats(const dsa_dims* dims, int32_t page_size, const int32_t* idx, int32_t* stats, void* stream);

/*
 * Forward indexer KL on the selected set (page "6.2 DSA Continued
 * Pre-Training: Warm-up and Sparse Stages", sparse stage; the analysis page,
 * Sec. 1.1 Eq. (4)): for every query row t with selection S_t (idx),
 *   P_s   = sum_h exp(sm_scale * q[t,h] . kv[s] - lse[t,h])   (the attention
 *           weights of all heads over S_t; lse from dsa_sparse_mla_attn)
 *   p_s   = P_s / sum_{s' in S_t} P_s'                         (L1 normalised)
 *   kl[t] = sum_{s in S_t} p_s (ln p_s - ln softmax_{S_t}(I[t,:])_s)
 * with I[t,s] = scores[b, i, s] (the index scores).  kl is [B, n_q] f32; a
 * row with an empty selection gets 0.  layout may be NULL (dense caches, as
 * in dsa_sparse_mla_attn) or a paged / variable-length layout (as in the
 * _paged calls; idx holds token indices).  The weights are recomputed from
 * q and kv on bf16 MFMA with fp32 accumulation; sums are fp32.
 */
int dsa_indexer_kl(const dsa_dims* dims, const dsa_paged_kv* layout, const uint16_t* q, const uint16_t* kv,
                   const int32_t* idx, const float* lse, const float* scores, int64_t ld, float sm_scale,
                   float* kl, void* stream);
/* dsa_forward (layout NULL) or dsa_forward_paged, plus kl [B, n_q] as in
 * dsa_indexer_kl for each chunk's selection and scores (the training forward
 * of the sparse stage).  lse and kl are required.  Equal, bit for bit, to the
 * forward followed by dsa_indexer_kl on its selection and scores. */
int dsa_forward_kl(const dsa_dims* dims, const dsa_paged_kv* layout, const uint8_t* q_idx, const float* q_scale,
                   const uint16_t* w_idx, const uint8_t* k_idx, const float* k_scale, const uint16_t* q,
                   const uint16_t* kv, float sm_scale, uint16_t* out, float* lse, int32_t* idx_out, float* kl,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * Masked MHA mode for short prefills (the technical report's Inference Costs
 * paragraph, forum translation Sec. 3: short prefills simulate DSA with a
 * masked MHA mode; the analysis page's Fig. 3 discussion; MHA and MQA as the
 * two equal forms of MLA, the analysis page around Fig. 7).
 *
 * MHA mode splits a latent row c_s (dim_qk dims) into its compressed part
 * c_s[0:dim_v] and its rope part c_s[dim_v:dim_qk] (shared by the heads).
 * Head h has the decompression matrices W_UK[h] [dim_nope, dim_v] and
 * W_UV[h] [dim_vh, dim_v]; its key of token s is
 * [W_UK[h] c_s[0:dim_v] | c_s[dim_v:]] and its value W_UV[h] c_s[0:dim_v].
 * The MHA query of head h is q_mha[b, i, h] = [q_nope (dim_nope) | q_rope
 * (dim_qk - dim_v)].  Masked MHA attention of row i (position p):
 *   z_s   = sm_scale * q_mha[b,i,h] . key_h(s)    over s <= p with mask bit set
 *   out   = sum_s softmax(z)_s value_h(s),   lse = log sum_s exp(z_s)
 * With the mask taken from the row's top-k selection this equals, up to
 * rounding, W_UV[h] applied to dsa_sparse_mla_attn's output for the absorbed
 * query [W_UK[h]^T q_nope | q_rope].
 *
 * Supported: (dim_nope, rope = dim_qk - dim_v, dim_vh) = (128, 64, 128) or
 * (32, 16, 32); dim_v a multiple of 64; heads <= 128; n_kv <= 65536.
 */

/* Selection bitmap: mask [B, ceil(n_kv / 32), n_q] uint32; bit r of word
 * (b, c, i) is set iff token 32c + r is in row i's list idx[b, i, 0:topk]
 * and visible to the row (32c + r <= p, < n_kv).  Every word is written. */
int dsa_selection_mask(const dsa_dims* dims, const int32_t* idx, uint32_t* mask, void* stream);

/* Per-head keys and values of latent rows s < n_rows (0 <= n_rows <= n_kv):
 *   k_mha [B, H, n_kv, dim_nope] bf16:  k_mha[b,h,s] = W_UK[h] kv[b,s,0:dim_v]
 *   v_mha [B, H, n_kv, dim_vh]   bf16:  v_mha[b,h,s] = W_UV[h] kv[b,s,0:dim_v]
 * w_uk [H, dim_nope, dim_v], w_uv [H, dim_vh, dim_v] bf16.  bf16 MFMA with
 * fp32 accumulation, rounded once to bf16.  Rows >= n_rows are not written. */
int dsa_mha_decompress(const dsa_dims* dims, int32_t dim_nope, int32_t dim_vh, const uint16_t* kv, const uint16_t* w_uk,
                       const uint16_t* w_uv, int32_t n_rows, uint16_t* k_mha, uint16_t* v_mha, void* stream);

/* Masked MHA attention.  q_mha [B, T, H, dim_nope + dim_qk - dim_v] bf16,
 * kv [B, S, dim_qk] (rope dims read), k_mha / v_mha as written by
 * dsa_mha_decompress (rows s < q_pos0 + n_q must hold finite values),
 * mask as written by dsa_selection_mask (any bit pattern is allowed: the
 * causal limit is applied as well).  out [B, T, H, dim_vh] bf16, lse
 * [B, T, H] f32 or NULL; a row with no visible selected key gets out = 0
 * and lse = -inf.  bf16 MFMA, fp32 accumulation and softmax. */
int dsa_masked_mha_attn(const dsa_dims* dims, int32_t dim_nope, int32_t dim_vh, const uint16_t* q_mha,
                        const uint16_t* kv, const uint16_t* k_mha, const uint16_t* v_mha, const uint32_t* mask,
                        float sm_scale, uint16_t* out, float* lse, void* stream);

/* Whole short-prefill path: indexer -> top-k -> selection mask (in chunks
 * of query rows, as dsa_forward) -> decompression of the rows s < q_pos0 +
 * n_q -> masked MHA attention.  Inputs as in dsa_forward plus q_mha, w_uk
 * and w_uv; idx_out [B, T, topk] or NULL receives the selection.  Equal, bit
 * for bit, to running the five calls one after the other.  ws must hold
 * dsa_masked_mha_workspace_size(dims, dim_nope, dim_vh) bytes (256-byte
 * aligned). */
size_t dsa_masked_mha_workspace_size(const dsa_dims* dims, int32_t dim_nope, int32_t dim_vh);
int dsa_masked_mha_forward(const dsa_dims* dims, int32_t dim_nope, int32_t dim_vh, const uint8_t* q_idx,
                           const float* q_scale, const uint16_t* w_idx, const uint8_t* k_idx, const float* k_scale,
                           const uint16_t* q_mha, const uint16_t* kv, const uint16_t* w_uk, const uint16_t* w_uv,
                           float sm_scale, uint16_t* out, float* lse, int32_t* idx_out, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * Opt-in device check of the inputs whose values the host cannot see (the
 * analysis page, Sec. 5.1: check valid lengths and the finiteness of scales
 * at kernel entry; odd scales and NaN destabilise the selection).  The
 * stage kernels never read outside their buffers whatever these values are
 * (lengths and page entries are clamped, NaN scores rank last); this call
 * reports them so a caller can reject a batch.  Asynchronous on `stream`:
 * it writes counts [8] int32 (device, 4-byte aligned, overwritten):
 *   counts[0]  q_scale [B, n_q] entries that are NaN, infinite or <= 0
 *   counts[1]  w_idx [B, n_q, H_I] bf16 entries that are NaN or infinite
 *   counts[2]  k_scale entries of the tokens a query row can see (dense:
 *              s < q_pos0 + n_q; paged: s < seq_lens[b]) that are NaN,
 *              infinite or <= 0
 *   counts[3]  idx [B, n_q, topk] entries that are neither -1 nor in
 *              [0, n_p) for their row
 *   counts[4]  idx rows not in the form dsa_topk writes (valid entries
 *              strictly ascending, then only -1): such a row may repeat an
 *              entry, which the attention would weigh twice
 *   counts[5]  seq_lens entries outside [n_q, n_kv] (layout given)
 *   counts[6]  page_table entries outside [0, num_pages) among the pages a
 *              sequence's tokens use (layout with a page table)
 *   counts[7]  0
 * layout: NULL (dense caches) or a paged / variable-length layout as in the
 * _paged calls.  Any of q_scale, w_idx, k_scale and idx may be NULL to skip
 * its check (w_idx needs idx_heads in [1, 64]; idx needs topk).
 */
int dsa_validate(const dsa_dims* dims, const dsa_paged_kv* layout, const float* q_scale, const uint16_t* w_idx,
                 const float* k_scale, const int32_t* idx, int32_t* counts, void* stream);

/* Status text, thread-local last error message, ABI version (major*100+minor). */
const char* dsa_status_string(int status);
const char* dsa_last_error(void);
int dsa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H_ */
