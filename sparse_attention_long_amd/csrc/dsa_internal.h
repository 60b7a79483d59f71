// Internal launch interface between the C ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

namespace dsa {

// One-time set-up per device that host threads may reach concurrently
// (kernel attributes, device properties): f runs once per device under
// std::call_once and its int result is kept for later calls.
constexpr int kMaxDevices = 64;
struct DeviceOnce {
  std::once_flag flag[kMaxDevices];
  int value[kMaxDevices] = {};
};
// Returns f()'s kept result for the current device, or `on_error` if the
// current device cannot be read or is beyond kMaxDevices.
template <class F>
int device_once(DeviceOnce& o, int on_error, F&& f) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return on_error;
  std::call_once(o.flag[dev], [&] { o.value[dev] = f(dev); });
  return o.value[dev];
}

// Cache layout.  Dense (both pointers null): sequence b's token s is row
// b * S + s of the caches and every sequence holds S tokens.  Otherwise
// sequence b holds len(b) = clamp(seq_lens[b], n_q_total, S) tokens, its
// query rows are its last n_q_total tokens, and with a page table its token
// s is pool row page_table[b * max_pages + s / page_size] * page_size +
// s % page_size (page entries clamped to [0, num_pages)).  Clamping keeps a
// bad device-side value from addressing memory outside the buffers.
struct PagedKV {
  const int32_t* seq_lens;     // [B] or null
  const int32_t* page_table;   // [B, max_pages] or null
  int page_size, max_pages, num_pages;
  int n_q_total;               // query rows per sequence (all chunks)
};

__device__ __forceinline__ int seq_len_of(const PagedKV& p, int b, int S) {
  return p.seq_lens ? min(max(p.seq_lens[b], p.n_q_total), S) : S;
}
// Absolute position of a launch's row 0 of sequence b, given the launch's
// pos0 (dense: the position itself; with seq_lens: the row offset within
// the sequence's query rows).
__device__ __forceinline__ int row_pos_base(const PagedKV& p, int b, int S, int pos0) {
  return p.seq_lens ? seq_len_of(p, b, S) - p.n_q_total + pos0 : pos0;
}
// Physical page of logical page j of sequence b (paged layouts only).
__device__ __forceinline__ int64_t page_of(const PagedKV& p, int b, int j) {
  const int e = p.page_table[(int64_t)b * p.max_pages + min(j, p.max_pages - 1)];
  return (int64_t)min(max(e, 0), p.num_pages - 1);
}
// Cache row of token s of sequence b.
__device__ __forceinline__ int64_t cache_row(const PagedKV& p, int b, int S, int s) {
  if (!p.page_table) return (int64_t)b * S + s;
  return page_of(p, b, s / p.page_size) * p.page_size + s % p.page_size;
}

// A span of query rows: rows [0, rows) of each of B sequences, where row i
// sits at absolute position row_pos_base(pk, b, S, pos0) + i.  Row-indexed
// tensors advance by `qrows_b` rows from one sequence to the next.
struct IndexerArgs {
  const uint8_t* q_idx;   // [B, qrows_b, HI, dI] e4m3
  const float* q_scale;   // [B, qrows_b]
  const uint16_t* w;      // [B, qrows_b, HI] bf16
  const uint8_t* k_idx;   // [B, S, dI] e4m3
  const float* k_scale;   // [B, S]
  float* scores;          // [B, sc_rows_b, ld]
  int64_t ld;
  int64_t qrows_b;
  int64_t sc_rows_b;
  int B, rows, pos0, S, HI, dI;
  PagedKV pk;             // k_idx / k_scale are pools when pk.page_table is set
};

struct TopkArgs {
  const float* scores;    // [B, sc_rows_b, ld]
  int32_t* idx;           // [B, idx_rows_b, k]
  int64_t ld;
  int64_t sc_rows_b;
  int64_t idx_rows_b;
  int B, rows, pos0, S, k;
  PagedKV pk;             // only the lengths are used
};

struct AttnArgs {
  const uint16_t* q;      // [B, qrows_b, H, Dk] bf16
  const uint16_t* kv;     // [B, S, Dk] bf16
  const int32_t* idx;     // [B, idx_rows_b, k]
  uint16_t* out;          // [B, qrows_b, H, Dv] bf16
  float* lse;             // [B, qrows_b, H] or null
  uint16_t* part_o;       // split partials [B*rows, nsplit, H, Dv] bf16, each normalised (nsplit > 1)
  float* part_lse;        // [B*rows, nsplit, H]
  int64_t qrows_b;        // row stride between sequences for q, out, lse
  int64_t idx_rows_b;     // row stride between sequences for idx
  int B, rows, S, H, Dk, Dv, k, nsplit;
  float sm_scale;
  PagedKV pk;             // kv is a pool when pk.page_table is set; idx holds token indices
};

// Kernel choice for the indexer: decode form (one row per wave, keys split
// across waves) for spans of at most this many rows per sequence.
constexpr int kIndexerDecodeMaxRows = 4;

hipError_t launch_indexer(const IndexerArgs& a, bool decode_form, hipStream_t st);
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);
// Split top-k for few long rows: each row's collection is spread over
// nparts workgroups whose candidates meet in a caller workspace of
// topk_split_bytes(rows_total, nparts) bytes; the selection is the same as
// launch_topk's.  nparts <= 1 runs launch_topk.
int topk_split_parts(int64_t rows_total, int S);
size_t topk_split_bytes(int64_t rows_total, int nparts);
hipError_t launch_topk_split(const TopkArgs& a, int nparts, void* ws, hipStream_t st);
hipError_t launch_sparse_mla(const AttnArgs& a, hipStream_t st);
// Indexer KL of each row over its selection: `at` as for the attention, with
// at.lse the attention's log-sum-exp (input), at.out unused.
struct KlArgs {
  AttnArgs at;
  const float* scores;    // [B, sc_rows_b, ld] index scores of the rows
  int64_t ld, sc_rows_b;
  float* kl;              // [B, qrows_b]
};
hipError_t launch_indexer_kl(const KlArgs& a, hipStream_t st);

// Locality counters of rows of selected token indices ([rows, k], k <= 2048).
hipError_t launch_gather_stats(const int32_t* idx, int32_t* stats, int64_t rows, int k, int page_size,
                               hipStream_t st);

// Masked MHA mode (short prefill).
// Selection bitmap: rows [0, rows) of a span whose row r is query row
// row0 + r (absolute position pos0 + row0 + r) of each sequence; its index
// list is idx[(b * idx_rows_b + r) * k ...].  Writes words (b, c, row0 + r)
// of mask [B, NC, T] for every c < NC.
struct MaskArgs {
  const int32_t* idx;
  uint32_t* mask;
  int64_t idx_rows_b;
  int B, rows, row0, T, S, k, pos0, NC;
};
// Per-head decompression of latent rows [0, n_rows): out[m][b, h, s, :] =
// W_m[h] . kv[b, s, 0:Dv] for m = 0 (keys, rows_w[0] dims) and 1 (values).
struct DecompArgs {
  const uint16_t* kv;         // [B, S, Dk]
  const uint16_t* w[2];       // [H, rows_w[m], Dv]
  uint16_t* out[2];           // [B, H, S_h, rows_w[m]]
  int rows_w[2];
  int B, S, H, Dk, Dv, n_rows, S_h;
};
struct MhaArgs {
  const uint16_t* q;          // [B, T, H, dn + dr]
  const uint16_t* kv;         // [B, S, Dk] (rope dims [Dv, Dk))
  const uint16_t* kh;         // [B, H, S_h, dn]
  const uint16_t* vh;         // [B, H, S_h, dvh]
  const uint32_t* mask;       // [B, NC, T]
  uint16_t* out;              // [B, T, H, dvh]
  float* lse;                 // [B, T, H] or null
  int B, T, S, S_h, H, Dk, Dv, pos0, NC;
  float sm_scale;
};
bool mha_dims_supported(int dn, int dr, int dvh, int Dv);
hipError_t launch_selection_mask(const MaskArgs& a, hipStream_t st);
hipError_t launch_mha_decompress(const DecompArgs& a, hipStream_t st);
hipError_t launch_masked_mha(const MhaArgs& a, int dn, int dr, int dvh, hipStream_t st);

// Device check of inputs (counts of bad values, see dsa_validate).  Any of
// q_scale, w, k_scale and idx may be null to skip its check; pk.seq_lens
// null means dense caches (then key scales are checked for the tokens
// s < q_pos0 + n_q that some query row can see).
constexpr int kValidateCounts = 8;
struct ValidateArgs {
  const float* q_scale;   // [B, n_q]
  const uint16_t* w;      // [B, n_q, HI] bf16
  const float* k_scale;   // [B, S] or a pool
  const int32_t* idx;     // [B, n_q, k]
  int32_t* counts;        // [kValidateCounts]
  int B, n_q, S, HI, k, q_pos0;
  PagedKV pk;
  int blocks_q, blocks_k, blocks_idx, blocks_seq;   // set by the launcher
};
hipError_t launch_validate(ValidateArgs a, hipStream_t st);

// Shape support checks (true if the kernels are built for these dims).
bool attn_dims_supported(int H, int Dk, int Dv);
int topk_max_kv();

// Per-token E4M3 quantisation of n_tokens rows of len values (dtype 0 f32,
// 1 bf16); token tok goes to output row (tok / group) * out_stride + out_off
// + tok % group of codes/scales.
hipError_t launch_quantize(const void* x, int dtype, int64_t n_tokens, int32_t len, int32_t group,
                           int64_t out_stride, int64_t out_off, uint8_t* codes, float* scales, hipStream_t st);
// Copy of n_rows bf16 rows of row_len (a multiple of 8) with the same row mapping.
hipError_t launch_copy_rows(const uint16_t* src, uint16_t* dst, int64_t n_rows, int32_t row_len, int32_t group,
                            int64_t out_stride, int64_t out_off, hipStream_t st);

}  // namespace dsa
