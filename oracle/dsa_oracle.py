"""CPU reference for the DeepSeek Sparse Attention (DSA) forward path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it, and it shares no code with the GPU library.

It is the plain definition of the method, evaluated directly in float64 with
numpy (a matrix product and a sort serve as library steps; nothing is blocked,
fused or reordered beyond what the definitions state).  Sources, all on the
page "DeepSeek-V3.2: sparse attention, scaled RL and synthetic agent
environments" (PaperTrace analysis of arXiv 2512.02556):

* Lightning indexer, Sec. 1.1 Eq. (1):
      I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s])
  over the tokens s that precede the query t.
* Fine-grained token selection, Sec. 1.1 (Eq. (4) defines the set):
      S_t = { s : I[t,s] in Top-k(I[t,:]) }
* Sparse attention, Sec. 1.1 Eq. (2): u_t = Attn(h_t, {c_s : s in S_t}); the
  index scores only choose the set and do not enter the attention weights;
  the softmax is taken over the selected set only (Sec. 5.2 Eq. (19)).
* MLA in MQA mode, Sec. 1.1 (and Fig. 7): every selected 576-d latent row is
  shared by all 128 query heads; keys are the whole row, values its first
  512 dims.
* Short rows select among min(k, t) positions (Sec. 5.1).

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
* "preceding" is inclusive: a query at absolute position p sees s <= p, so a
  row has n_p = min(p + 1, S) candidates and m_p = min(k, n_p) selections.
* FP8 is OCP E4M3 (E4M3FN) with one positive fp32 scale per token; the
  quantised value is code * scale.  Eq. (1) is evaluated on those values.
* No extra constant (1/sqrt(d) etc.) in Eq. (1).
* Ties at the top-k cutoff go to the lower index; the selected set is
  reported in ascending index order padded with -1 to k entries.  NaN ranks
  below every number; -0.0 equals +0.0.
* Attention logits are sm_scale * (q . c_s) over all Dk dims; values are
  c_s[0:Dv].
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------- formats
def _e4m3_table() -> np.ndarray:
    """Value of every OCP FP8 E4M3FN byte (OCP 8-bit Floating Point
    Specification v1.0, E4M3: sign, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent 0 is subnormal; S.1111.111 is NaN; no infinities)."""
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = s * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            t[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


E4M3_VALUES = _e4m3_table()


def e4m3_decode(codes) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def bf16_decode(bits) -> np.ndarray:
    """bfloat16 bit pattern -> float64 (bf16 is the top half of a float32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def dequant_e4m3(codes, scales) -> np.ndarray:
    """value = decoded code * per-token scale (exact in float64)."""
    v = e4m3_decode(codes)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    return v * s.reshape(s.shape + (1,) * (v.ndim - s.ndim))


# ----------------------------------------------------------------- quantisation
def quantize_e4m3_tokens(x):
    """Per-token FP8 quantisation (the FP8 indexer inputs of Sec. 1.1, in the
    format and scale granularity read into the pages here): scale =
    amax / 448 in float32 (1 for an all-zero token); each value is divided by
    the scale in float32 and rounded to the nearest E4M3FN value, ties to the
    even code, with magnitudes of 448 and above saturating to 448.  The sign
    of the quotient is kept (a -0.0 quotient gives code 0x80).

    x: [..., token_len] values; returns (codes uint8 [..., token_len],
    scales float32 [...])."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    y = (x32 / scale[..., None]).astype(np.float32)
    a = np.abs(y).astype(np.float64)
    vals = E4M3_VALUES[:0x7F]                     # codes 0x00..0x7E, increasing, 0 .. 448
    hi = np.clip(np.searchsorted(vals, a), 1, 0x7E)
    lo = hi - 1
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    code = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a >= 448.0, 0x7E, code)
    code = code.astype(np.uint8) | (np.signbit(y).astype(np.uint8) << np.uint8(7))
    return code.astype(np.uint8), scale


def cache_append(k_cache, k_scale_cache, kv_cache, k_new, kv_new, pos0: int):
    """The decode cache update: the new tokens of every sequence (axis 1 of
    k_new / kv_new) are quantised (keys) or copied (latents) into rows
    pos0 .. pos0 + n - 1 of the caches; returns updated copies."""
    kc, ks, kv = np.array(k_cache), np.array(k_scale_cache), None if kv_cache is None else np.array(kv_cache)
    codes, scales = quantize_e4m3_tokens(k_new)
    n = codes.shape[1]
    kc[:, pos0:pos0 + n] = codes
    ks[:, pos0:pos0 + n] = scales
    if kv is not None:
        kv[:, pos0:pos0 + n] = kv_new
    return kc, ks, kv


# ----------------------------------------------------------------- shapes
def n_candidates(p: int, n_kv: int) -> int:
    """n_p = min(p + 1, S): inclusive causal row length at absolute position p."""
    return min(p + 1, n_kv)


def n_selected(p: int, n_kv: int, k: int) -> int:
    """m_p = min(k, n_p) (short rows select everything they have)."""
    return min(k, n_candidates(p, n_kv))


# ----------------------------------------------------------------- Eq. (1)
def indexer_row(q_t: np.ndarray, w_t: np.ndarray, k_all: np.ndarray, p: int) -> np.ndarray:
    """Index scores of one query row.

    q_t: [H_I, d_I] real-valued indexer queries of token t.
    w_t: [H_I] head weights of token t.
    k_all: [S, d_I] real-valued indexer keys.
    p: absolute position of the query.
    Returns float32 [n_p]: I[t, s] for s = 0..n_p-1, computed in float64 as
    sum_j w[t,j] * max(0, q[t,j] . k[s]) and rounded once to float32."""
    n = n_candidates(p, k_all.shape[0])
    q = np.asarray(q_t, dtype=np.float64)
    k = np.asarray(k_all[:n], dtype=np.float64)
    w = np.asarray(w_t, dtype=np.float64)
    dots = k @ q.T                          # [n, H_I]: q[t,j] . k[s]
    relu = np.maximum(dots, 0.0)
    return (relu @ w).astype(np.float32)


def indexer_scores(q_idx, w_idx, k_idx, q_pos0: int) -> list:
    """All rows of one sequence: q_idx [T, H_I, d_I], w_idx [T, H_I],
    k_idx [S, d_I].  Returns a list of float32 rows (row i has n_p entries)."""
    return [indexer_row(q_idx[i], w_idx[i], k_idx, q_pos0 + i) for i in range(q_idx.shape[0])]


# ----------------------------------------------------------------- Top-k
def topk_row(scores: np.ndarray, k: int) -> np.ndarray:
    """Top-k of one score row (all entries are candidates).

    Order: larger score first; NaN below every number; -0.0 == +0.0; equal
    scores go to the lower index.  Returns int32 [k]: the chosen indices in
    ascending order, then -1 padding."""
    x = np.asarray(scores, dtype=np.float32).astype(np.float64)
    n = x.shape[0]
    m = min(k, n)
    nan = np.isnan(x)
    val = np.where(nan, 0.0, x) + 0.0       # + 0.0 maps -0.0 to +0.0
    idx = np.arange(n)
    order = np.lexsort((idx, -val, nan))     # primary: not-NaN first; then value desc; then index asc
    chosen = np.sort(order[:m])
    out = np.full(k, -1, dtype=np.int32)
    out[:m] = chosen
    return out


# ----------------------------------------------------------------- Eq. (2)/(19)
def sparse_mla_row(q_t: np.ndarray, kv: np.ndarray, sel: np.ndarray, sm_scale: float, dim_v: int,
                   return_weights: bool = False):
    """MQA-mode attention of one query token over the selected latent rows.

    q_t: [H, Dk] absorbed per-head queries; kv: [S, Dk] latent rows (keys are
    whole rows, values their first dim_v dims); sel: selected row indices
    (entries < 0 are padding and skipped).  Softmax is over the selected set
    only.  Returns o [H, dim_v] and lse [H] (natural log of the softmax
    denominator including the max), in float64."""
    s = np.asarray(sel)
    s = s[s >= 0]
    q = np.asarray(q_t, dtype=np.float64)
    c = np.asarray(kv, dtype=np.float64)[s]           # [m, Dk]
    if s.size == 0:
        o = np.zeros((q.shape[0], dim_v))
        lse = np.full(q.shape[0], -np.inf)
        return (o, lse, np.zeros((q.shape[0], 0))) if return_weights else (o, lse)
    z = sm_scale * (q @ c.T)                          # [H, m]
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    den = e.sum(axis=1, keepdims=True)
    p = e / den
    o = p @ c[:, :dim_v]
    lse = (zmax + np.log(den))[:, 0]
    return (o, lse, p) if return_weights else (o, lse)


# ----------------------------------------------------------------- whole path
def dsa_row(q_idx_t, w_t, k_idx, q_t, kv, p: int, k: int, sm_scale: float, dim_v: int):
    """One query row through indexer -> top-k -> sparse attention.
    Returns (scores float32 [n_p], sel int32 [k], o [H, dim_v], lse [H])."""
    sc = indexer_row(q_idx_t, w_t, k_idx, p)
    sel = topk_row(sc, k)
    o, lse = sparse_mla_row(q_t, kv, sel, sm_scale, dim_v)
    return sc, sel, o, lse


# ----------------------------------------------------------------- paged / variable-length caches
# The analysis page, Sec. 5.1: rows of one batch have their own context length
# (per-sequence lengths limit each row to min(k, t) candidates), the selected
# entries of a row may sit in a few contiguous cache pages or be spread over
# many, and a profiler should count the distinct pages, the contiguous runs
# and the hits per page of a row's selection.
def paged_gather(pool, page_row, page_size: int, n: int) -> np.ndarray:
    """The first n logical tokens of one sequence from a page pool (axis 0 =
    physical token slot): logical token s lives in slot
    page_row[s // page_size] * page_size + s % page_size."""
    s = np.arange(n)
    slots = np.asarray(page_row, dtype=np.int64)[s // page_size] * page_size + s % page_size
    return np.asarray(pool)[slots]


def varlen_positions(seq_len: int, n_q: int) -> list:
    """Absolute positions of the n_q query rows of a sequence with seq_len
    cached tokens: its last n_q tokens (decode: n_q = 1, p = seq_len - 1)."""
    return [seq_len - n_q + i for i in range(n_q)]


def gather_stats(sel, page_size: int):
    """Locality of one row's selection (padding < 0 skipped): the number of
    distinct cache pages it touches, the number of maximal runs of
    consecutive token indices, and the largest number of selected tokens on
    one page.  An empty selection gives (0, 0, 0)."""
    s = np.asarray(sel, dtype=np.int64)
    s = np.sort(s[s >= 0])
    if s.size == 0:
        return 0, 0, 0
    pages, hits = np.unique(s // page_size, return_counts=True)
    runs = 1 + int(np.count_nonzero(np.diff(s) != 1))
    return int(pages.size), runs, int(hits.max())


# ----------------------------------------------------------------- indexer KL on the selected set
# Page "6.2 DSA Continued Pre-Training: Warm-up and Sparse Stages" (Stage 2)
# and the analysis page, Sec. 1.1 Eq. (4): the indexer is trained towards
# the main attention on the selected set.  The target p sums the attention
# weights of all heads and L1-normalises along the sequence; the loss of a
# query is KL(p_{t,S_t} || Softmax(I_{t,S_t})).
def indexer_kl_row(q_t, kv, sel, scores, sm_scale: float, dim_v: int):
    """KL divergence of one query row.

    q_t [H, Dk], kv [S, Dk] latent rows, sel: selected token indices (entries
    < 0 skipped), scores: the row's index scores I[t, s] (indexable by s).
    p_s = sum_h P[h, s] / sum_{h, s'} P[h, s'] with P the sparse attention
    weights of Eq. (19); q = softmax of I over the selected set.  Returns
    sum_s p_s (ln p_s - ln q_s) in float64 (0 for an empty selection)."""
    s = np.asarray(sel)
    s = s[s >= 0]
    if s.size == 0:
        return 0.0
    _, _, P = sparse_mla_row(q_t, kv, s, sm_scale, dim_v, return_weights=True)   # [H, m]
    agg = P.sum(axis=0)
    p = agg / agg.sum()
    i_sel = np.asarray(scores, dtype=np.float64)[s]
    i_max = i_sel.max()
    log_q = i_sel - (i_max + np.log(np.exp(i_sel - i_max).sum()))
    nz = p > 0
    return float((p[nz] * (np.log(p[nz]) - log_q[nz])).sum())


# ----------------------------------------------------------------- masked MHA mode (short prefill)
# The analysis page, the MQA-mode discussion with Fig. 7: MLA has two
# algebraically equal forms.  MHA mode decompresses each latent row into
# per-head keys and values; MQA mode folds the decompression matrices into
# the query so that every head reads the shared latent row.  The technical
# report's Inference Costs paragraph (forum translation, Sec. 3) and the
# analysis page's Fig. 3 discussion: short prefills use a masked MHA mode
# that simulates DSA, i.e. dense causal attention in MHA mode in which the
# keys outside the row's top-k set are masked out.
#
# Readings (the pages give no per-head sizes for MHA mode): a latent row is
# [compressed part (dim_v dims) | rope part (Dk - dim_v dims)]; head h has
# keys [W_UK[h] c | rope] and values W_UV[h] c, where c is the compressed
# part and the rope part is shared by all heads; the MHA query of head h is
# [q_nope (dn dims) | q_rope (Dk - dim_v dims)].
def mha_decompress(kv, w_uk, w_uv, dim_v: int):
    """MHA-mode keys and values of latent rows kv [n, Dk].
    w_uk [H, dn, dim_v], w_uv [H, dvh, dim_v].  Returns k_nope [H, n, dn]
    with k_nope[h, s] = W_UK[h] c_s, v [H, n, dvh] with v[h, s] = W_UV[h] c_s,
    and rope [n, Dk - dim_v] (float64)."""
    c = np.asarray(kv, dtype=np.float64)
    comp = c[:, :dim_v]
    k_nope = np.matmul(comp[None], np.asarray(w_uk, dtype=np.float64).transpose(0, 2, 1))
    v = np.matmul(comp[None], np.asarray(w_uv, dtype=np.float64).transpose(0, 2, 1))
    return k_nope, v, c[:, dim_v:]


def selection_mask(sel, n_keys: int) -> np.ndarray:
    """Boolean [n_keys]: True at the selected token indices (entries < 0 or
    >= n_keys are ignored)."""
    m = np.zeros(n_keys, dtype=bool)
    s = np.asarray(sel, dtype=np.int64)
    m[s[(s >= 0) & (s < n_keys)]] = True
    return m


def masked_mha_row(q_t, kv, w_uk, w_uv, sel, p: int, sm_scale: float, dim_v: int, kvh=None):
    """Masked MHA-mode attention of one query row at absolute position p.

    q_t [H, dn + dr] (decompressed-key dims first, then the rope dims);
    kv [S, Dk] latent rows.  Every key s <= p (s < S) is scored, keys outside
    the selection get -inf, and the softmax runs over the row:
        z[h, s] = sm_scale * (q_nope[h] . W_UK[h] c_s + q_rope[h] . rope_s)
        out[h]  = sum_s softmax(z[h])_s W_UV[h] c_s
    Returns out [H, dvh] and lse [H] (float64); a row with no selected key
    gets out = 0 and lse = -inf.  kvh: mha_decompress(kv[:m], ...) for some
    m >= min(p + 1, S), to share one decompression between rows."""
    q = np.asarray(q_t, dtype=np.float64)
    H, dn = q.shape[0], np.asarray(w_uk).shape[1]
    n = min(p + 1, np.asarray(kv).shape[0])
    if kvh is None:
        kvh = mha_decompress(np.asarray(kv)[:n], w_uk, w_uv, dim_v)
    k_nope, v, rope = kvh[0][:, :n], kvh[1][:, :n], kvh[2][:n]
    keep = selection_mask(sel, n)
    dvh = v.shape[2]
    if not keep.any():
        return np.zeros((H, dvh)), np.full(H, -np.inf)
    z = sm_scale * (np.einsum("hd,hsd->hs", q[:, :dn], k_nope) + q[:, dn:] @ rope.T)   # [H, n]
    z = np.where(keep[None, :], z, -np.inf)
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    den = e.sum(axis=1, keepdims=True)
    out = np.einsum("hs,hsd->hd", e / den, v)
    return out, (zmax + np.log(den))[:, 0]
