// Lightning indexer on FP8 MFMA (page "DeepSeek-V3.2: sparse attention,
// scaled RL and synthetic agent environments", Sec. 1.1, Eq. (1)):
//
//   I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s])
//
// With FP8 values q[t,j] = qs[t] * qhat[t,j], k[s] = ks[s] * khat[s] and
// positive per-token scales, ReLU(qs*ks*x) = qs*ks*ReLU(x), so
//
//   I[t,s] = ks[s] * sum_j (w[t,j]*qs[t]) * ReLU(qhat[t,j] . khat[s]).
//
// The dot products qhat . khat run on v_mfma_scale_f32_16x16x128_f8f6f4
// (16 heads x 16 keys x 128 dims per instruction: d_I = 128 is one K step).
// Heads are the M dimension so that the head sum is mostly lane-local: each
// lane holds 4 heads of one key per instruction, and the remaining sum over
// the four 16-lane rows is a reduce-scatter with two permlane swaps.
//
// The ReLU is split as ReLU(x) = (|x| + x) / 2.  With the folded weights
// w'[j] = w[t,j]*qs[t]/2,
//
//   I[t,s] / ks[s] = sum_j w'[j] |d_j| + sum_j w'[j] d_j,   d_j = qhat[t,j] . khat[s],
//
// where the first sum is one fma per head (the abs is a free source
// modifier) and the second is linear in the key: v[t] . khat[s] with
// v[t] = sum_j w'[j] qhat[t,j].  Per query row, v is split into e4m3
// residual levels (kLinLevels of them, each with an E8M0 scale per MFMA
// scale block of 32 values, each level leaving at most 1/16 of the previous
// residual), and one extra MFMA per key tile yields every level's dot
// product.  That halves the VALU work per score.  Each wave then issues a
// step's MFMAs back to back and its epilogue after them, so the two waves
// on a SIMD alternate between the matrix core and the VALU.
//
// Two work shapes:
//  * prefill: a wave keeps the A operands (q) of 2 query rows in registers
//    and streams pairs of 16-key tiles; the 4 (row, tile) partials are
//    reduce-scattered so each 16-lane row ends with 16 scores of one query.
//    Both prefill kernels (keys staged in LDS, or read directly for paged
//    caches and d_I < 128) share the per-tile arithmetic above and give
//    bit-identical scores.
//  * decode: a wave keeps one row's q and streams 4 key tiles per step; the
//    reduce-scatter leaves 64 consecutive keys' scores, one per lane.  A
//    wave sees only 512 keys, too few to pay for the level tile's set-up,
//    so this form applies the ReLU directly (same value, other rounding).
#include <climits>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kMaxHeadTiles = 4;   // H_I <= 64

// 16 bytes of a row of FP8 codes at byte offset `off` (zero if off >= len).
// Branch-free: the address is clamped inside the row and the value masked.
__device__ __forceinline__ u32x4 load16_or_zero(const uint8_t* row, int off, int len, bool ok) {
  const bool in = ok && off < len;
  const u32x4 x = *(const u32x4*)(row + min(off, len - 16));
  const u32x4 z = {0u, 0u, 0u, 0u};
  return in ? x : z;
}

// A operand: 16 heads x 128 bytes of one query row (zero outside H_I/d_I).
// Lane l holds head 16*ht + l%16, bytes [32*(l/16), 32*(l/16) + 32).
__device__ __forceinline__ v8i load_q_tile(const IndexerArgs& a, int b, int i, int ht, int lane) {
  const int h = ht * 16 + (lane & 15);
  const int off = 32 * (lane >> 4);
  const bool ok = i < a.rows && h < a.HI;
  const uint8_t* row = a.q_idx + (((int64_t)b * a.qrows_b + min(i, a.rows - 1)) * a.HI + min(h, a.HI - 1)) * a.dI;
  const u32x4 lo = load16_or_zero(row, off, a.dI, ok), hi = load16_or_zero(row, off + 16, a.dI, ok);
  return (v8i){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Streaming form of the B operand for the key loops.  A tile is 16 keys
// sbase .. sbase+15 (sbase wave-uniform); lane l reads key sbase + l%16,
// bytes [lane_off, lane_off + 32) where lane_off = min(32*(lane/16), d_I-16),
// and `dmask` says whether the lane's K bytes exist (d_I < 128 pads with
// zero).  Keys at or beyond S read key S-1 instead; their results are never
// stored (each score column depends only on its own key), so no zeroing is
// needed.
//
// Paged caches: a wave's key range [k_begin, k_end) spans at most 64 pages;
// lane j holds the physical page of logical page k_begin/P + j, and a tile
// (16-aligned, page sizes are multiples of 64) lies in one page, so its page
// comes from one lane read.
template <bool kFullD>
struct KeyStream {
  const uint8_t* kb;      // dense: the sequence's keys; paged: the pool
  const float* sb;        // the matching key scales
  int dI, smax, lane_off;
  bool lo_ok, hi_ok;
  // paging
  bool paged;
  int psz, pfirst, pent;
  __device__ __forceinline__ void init(const IndexerArgs& a, int b, int lane, int k_begin) {
    paged = a.pk.page_table != nullptr;
    kb = a.k_idx + (paged ? 0 : (int64_t)b * a.S * a.dI);
    sb = a.k_scale + (paged ? 0 : (int64_t)b * a.S);
    dI = a.dI;
    smax = a.S - 1;
    const int off = 32 * (lane >> 4);
    lane_off = min(off, a.dI - 16);
    lo_ok = off < a.dI;
    hi_ok = off + 16 < a.dI;
    psz = paged ? a.pk.page_size : 1;
    pfirst = paged ? k_begin / psz : 0;
    pent = paged ? (int)page_of(a.pk, b, pfirst + lane) : 0;
  }
  // Cache row of key sbase + off (sbase wave-uniform, the tile in one page).
  __device__ __forceinline__ int64_t row(int sbase, int off) const {
    const int sb0 = min(sbase, smax);
    const int s = min(sbase + off, smax);
    if (!paged) return s;
    const int pg = __builtin_amdgcn_readlane(pent, min(sb0 / psz - pfirst, 63));
    return (int64_t)pg * psz + s % psz;
  }
  __device__ __forceinline__ v8i load(int sbase, int kl) const {
    const uint8_t* p = kb + row(sbase, kl) * dI + lane_off;
    if constexpr (kFullD) {   // d_I = 128: every lane's 32 bytes exist
      const u32x4 lo = *(const u32x4*)p;
      const u32x4 hi = *(const u32x4*)(p + 16);
      return (v8i){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    const u32x4 lo = *(const u32x4*)p;
    const u32x4 hi = *(const u32x4*)(p + (hi_ok ? 16 : 0));
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 l = lo_ok ? lo : z, h = hi_ok ? hi : z;
    return (v8i){(int)l[0], (int)l[1], (int)l[2], (int)l[3], (int)h[0], (int)h[1], (int)h[2], (int)h[3]};
  }
  // Scale of key sbase + off (zero past S).
  __device__ __forceinline__ float scale(int sbase, int off) const {
    const float v = sb[row(sbase, off)];
    return sbase + off <= smax ? v : 0.f;
  }
};

// Folded head weights w[t,j]*qs[t]*fold for the 4 heads (per head tile)
// this lane sees in the MFMA result: head 16*ht + 4*(lane/16) + r.
__device__ __forceinline__ void load_weights(const IndexerArgs& a, int b, int i, int lane, float fold,
                                             float (&wq)[kMaxHeadTiles][4]) {
  // Branch-free: clamped indices, then masks, so all loads are in flight at once.
  const bool row_ok = i < a.rows;
  const int64_t row = (int64_t)b * a.qrows_b + min(i, a.rows - 1);
  const float qs = row_ok ? a.q_scale[row] : 0.f;
  const uint16_t* wr = a.w + row * a.HI;
  if (a.HI % 4 == 0 && (reinterpret_cast<uintptr_t>(a.w) & 7) == 0) {
    // the 4 heads of a lane are consecutive: one 8-byte load per head tile
#pragma unroll
    for (int ht = 0; ht < kMaxHeadTiles; ++ht) {
      const int h0 = 16 * ht + 4 * (lane >> 4);
      const bool ok = row_ok && h0 < a.HI;
      const uint2 v = *(const uint2*)(wr + min(h0, a.HI - 4));
      const float w4[4] = {__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                           __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u)};
#pragma unroll
      for (int r = 0; r < 4; ++r) wq[ht][r] = ok ? w4[r] * qs * fold : 0.f;
    }
    return;
  }
#pragma unroll
  for (int ht = 0; ht < kMaxHeadTiles; ++ht)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 16 * ht + 4 * (lane >> 4) + r;
      const float wv = bf16_to_f32(wr[min(h, a.HI - 1)]);
      wq[ht][r] = (row_ok && h < a.HI) ? wv * qs * fold : 0.f;
    }
}

// max(x, 0) as one integer max on the bit pattern: negative floats (and
// -0.0) are negative as int32, positive ones keep their bits.  fmaxf would
// first canonicalise the MFMA result (one more VALU op per element).
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Decode form: one query row and four key tiles; for u = 0..3 this lane's
// share of sum_h wq[h] * ReLU(qhat_h . khat) for key tile kt[u], in the
// fixed order ht = 0..NHT-1, r = 0..3.  With few keys per wave the level
// tile of the prefill form would not pay for its set-up, so this form
// keeps the ReLU (weights folded as w[t,j]*qs[t]).  Each result's epilogue
// runs four MFMAs after it was issued (1 MFMA : 8 VALU).
template <int NHT>
__device__ __forceinline__ void tile_partials_relu(const v8i* qa, const float (*wq)[4], const v8i* const (&kt)[4],
                                                   float (&acc)[4]) {
  v4f d[NHT][4];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int u = 0; u < 4; ++u) d[ht][u] = mfma_fp8_16x16x128(qa[ht], *kt[u]);
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = 0.f;
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[u] = fmaf(wq[ht][r], relu_bits(d[ht][u][r]), acc[u]);
  __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);
#pragma unroll
  for (int k = 0; k < 4 && k < 4 * NHT; ++k) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
  for (int k = 4; k < 4 * NHT; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);
}

// ---- Prefill form: the ReLU split and the level tile ----
//
// The extra MFMA's A operand has 16 rows = 2 slots x 8 levels: row
// rho = 4*G + j (G = rho/4, j = rho%4) is slot j/2, level 2*G + j%2.  A
// result lane in 16-lane row G thus holds, for its key, levels 2G and 2G+1
// of slot 0 (elements 0, 1) and of slot 1 (elements 2, 3); the reduce-scatter
// over the four rows that already sums the head partials also sums the
// levels.  Levels kLinLevels..7 are zero rows.  Query row i of a prefill
// span takes slot i % 2 (waves start at even rows), in both prefill kernels.
constexpr int kLinLevels = 6;
constexpr int kLinScratch = 2 * 8 * 128 + 2 * 8 * 4;   // LDS per wave: codes [slot][level][128 B], E8M0 [slot][level][4]

struct LinOp {
  v8i a;    // codes of row lane%16, K bytes [32*(lane/16), +32)
  int sc;   // their E8M0 block scale
};

// Inputs of v for the query rows of the two slots.  Lane l covers the 16
// code bytes [16*(l%8), +16) of the heads 16*ht + 4*(l/16) + 2*((l/8)%2) + j
// (ht < NHT, j < 2): heads whose folded weights the lane already holds from
// load_weights (wq[ht][2*((l/8)%2) + j]).  All loads are issued at once,
// ahead of the q tiles; a slot whose row lies outside [0, rows) loads zeros.
template <int NHT>
struct LinLoads {
  u32x4 x[2][2 * NHT];
};

template <int NHT>
__device__ __forceinline__ void lin_load(const IndexerArgs& a, int b, int r0, int r1, int lane, LinLoads<NHT>& ld) {
  const int c = lane & 7;
  const int hbase = 4 * (lane >> 4) + 2 * ((lane >> 3) & 1);
#pragma unroll
  for (int sl = 0; sl < 2; ++sl) {
    const int i = sl ? r1 : r0;
    const bool row_ok = i >= 0 && i < a.rows;
    const int64_t row = (int64_t)b * a.qrows_b + min(max(i, 0), a.rows - 1);
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int h = 16 * ht + hbase + j;
        const bool ok = row_ok && h < a.HI;
        ld.x[sl][2 * ht + j] = load16_or_zero(a.q_idx + (row * a.HI + min(h, a.HI - 1)) * a.dI, 16 * c, a.dI, ok);
      }
  }
}

// v of slot sl (weights wq of that row), partly reduced.  Lane l first
// sums its 2*NHT heads over 16 values of K, then the sums are combined
// over lane bits 5 and 4: lane l ends with the sum over the heads j with
// (j/2) % 2 == (l/8) % 2, for k = 16*(l%8) + 4*(l/16) + t, t = 0..3.  Lanes
// l and l^8 hold the two halves of each total.
template <int NHT>
__device__ __forceinline__ void lin_half_sums(const LinLoads<NHT>& ld, int sl, const float (&wq)[kMaxHeadTiles][4],
                                              int lane, float (&out)[4]) {
  const bool odd = (lane & 8) != 0;
  float p[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) p[t] = 0.f;
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float w_lo = wq[ht][j], w_hi = wq[ht][2 + j];   // values, not lvalues: keeps wq in registers
      const float wv = odd ? w_hi : w_lo;
      const u32x4& x = ld.x[sl][2 * ht + j];
#pragma unroll
      for (int dw = 0; dw < 4; ++dw) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)x[dw], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)x[dw], true);
        p[4 * dw + 0] = fmaf(wv, lo[0], p[4 * dw + 0]);
        p[4 * dw + 1] = fmaf(wv, lo[1], p[4 * dw + 1]);
        p[4 * dw + 2] = fmaf(wv, hi[0], p[4 * dw + 2]);
        p[4 * dw + 3] = fmaf(wv, hi[1], p[4 * dw + 3]);
      }
    }
  // sum over lane bit 5 (p[t] stays in lanes < 32, p[t+8] in lanes >= 32),
  // then over bit 4 (rows 0, 2 keep the first four, rows 1, 3 the last four)
  float r1[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) r1[t] = reduce_halves(p[t], p[t + 8]);
#pragma unroll
  for (int t = 0; t < 4; ++t) out[t] = reduce_rows16(r1[t], r1[t + 4]);
}

// Level-tile operand from the loads of lin_load and the rows' folded
// weights (slot 0: row r0 with wq0, slot 1: row r1 with wq1).  `scratch`
// is kLinScratch bytes of LDS owned by this wave (16-byte aligned).
template <int NHT>
__device__ __forceinline__ LinOp lin_operand(const LinLoads<NHT>& ld, const float (&wq0)[kMaxHeadTiles][4],
                                             const float (&wq1)[kMaxHeadTiles][4], int lane, uint8_t* scratch) {
  float h0[4], h1[4];
  lin_half_sums<NHT>(ld, 0, wq0, lane, h0);
  lin_half_sums<NHT>(ld, 1, wq1, lane, h1);
  // Sum over lane bit 3, keeping slot 0 in lanes with bit 3 clear and slot
  // 1 in the others: lane l then holds v[slot][16*(l%8) + 4*(l/16) + t].
  const bool odd = (lane & 8) != 0;
  float v[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const float keep = odd ? h1[t] : h0[t], send = odd ? h0[t] : h1[t];
    v[t] = keep + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), 0x128, 0xF, 0xF, false));   // row_ror:8
  }
  const int slot = odd ? 1 : 0;
  uint32_t* codes = (uint32_t*)scratch;        // [slot][level][32 dwords]
  uint8_t* scl = scratch + 2 * 8 * 128;        // [slot][level][4 blocks]
  const int dw = 4 * (lane & 7) + (lane >> 4);   // dword holding k = 16*(l%8) + 4*(l/16) + 0..3
  // Its MFMA scale block: block sb holds the k with 2*((k%32)/16) + k/64 == sb,
  // and the scale of (row rho, sb) comes from lane 16*sb + rho.
  const int blk = 2 * (lane & 1) + ((lane >> 2) & 1);
#pragma unroll
  for (int lev = 0; lev < 8; ++lev) {
    uint32_t code = 0u, e8 = 127u;
    if (lev < kLinLevels) {
      // block max over the 8 lanes of (slot, block): lane bits 1, 4 and 5
      float mx = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
      mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mx), 0x4E, 0xF, 0xF, false)));   // quad_perm 2,3,0,1
      mx = max_halves(max_rows16(mx));
      // scale 2^(E-7-127): the block max lands in [128, 256), below the e4m3 limit
      const uint32_t E = __float_as_uint(mx) >> 23;
      const bool zero = E < 30u;   // nothing left worth a level (below 2^-97)
      e8 = zero ? 127u : E - 7u;
      const float down = zero ? 0.f : __uint_as_float((261u - E) << 23);
      const float up = zero ? 0.f : __uint_as_float((E - 7u) << 23);
      int c2 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0] * down, v[1] * down, 0, false);
      c2 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2] * down, v[3] * down, c2, true);
      const auto q01 = __builtin_amdgcn_cvt_pk_f32_fp8(c2, false);
      const auto q23 = __builtin_amdgcn_cvt_pk_f32_fp8(c2, true);
      // the residual is exact: the level value lies within a factor 2 of v
      v[0] = fmaf(-q01[0], up, v[0]);
      v[1] = fmaf(-q01[1], up, v[1]);
      v[2] = fmaf(-q23[0], up, v[2]);
      v[3] = fmaf(-q23[1], up, v[3]);
      code = (uint32_t)c2;
    }
    codes[(slot * 8 + lev) * 32 + dw] = code;
    scl[(slot * 8 + lev) * 4 + blk] = (uint8_t)e8;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int rho = lane & 15, gk = lane >> 4;
  const int rs = (rho >> 1) & 1, rl = 2 * (rho >> 2) + (rho & 1);
  const u32x4 lo = *(const u32x4*)(codes + (rs * 8 + rl) * 32 + 8 * gk);
  const u32x4 hi = *(const u32x4*)(codes + (rs * 8 + rl) * 32 + 8 * gk + 4);
  LinOp op;
  op.a = (v8i){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  op.sc = scl[(rs * 8 + rl) * 4 + gk];
  return op;
}

// Four partial head sums: for u = 0..3, the MFMA products of query operand
// set qa[u] (NHT head tiles) with key tile kt[u], followed by this lane's
// share of sum_h wq[u][h] * |dot| + (linear term), in the fixed order: the
// level pair first, then ht = 0..NHT-1, r = 0..3.  u = 2*q + t: query row q
// of the wave's pair (slot q), key tile t (kt = {t0, t1, t0, t1}); one level
// MFMA per key tile.
template <int NHT>
__device__ __forceinline__ void tile_partials(const v8i* const (&qa)[4], const float (*const (&wq)[4])[4],
                                              const v8i* const (&kt)[4], const LinOp& lin, float (&acc)[4]) {
  constexpr int NL = 2;
  v4f e[NL];
#pragma unroll
  for (int t = 0; t < NL; ++t) e[t] = mfma_fp8_16x16x128_sa(lin.a, lin.sc, *kt[t]);
  v4f d[NHT][4];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int u = 0; u < 4; ++u) d[ht][u] = mfma_fp8_16x16x128(qa[u][ht], *kt[u]);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const v4f& x = e[u & 1];
    acc[u] = (u >> 1) ? x[2] + x[3] : x[0] + x[1];
  }
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[u] = fmaf(wq[u][ht][r], fabsf(d[ht][u][r]), acc[u]);
  // schedule: pending LDS reads (the next step's operands, if any) first,
  // then every MFMA back to back, then the epilogue.  With two waves per
  // SIMD the waves fall into alternation, one streaming MFMAs while the
  // other runs its VALU epilogue; in a step-body probe this beat any
  // interleave of MFMA and VALU within a wave by 12-15%.
  __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, NL + 4 * NHT, 0);
  __builtin_amdgcn_sched_group_barrier(0x002, 96, 0);
}

// Workgroup -> (query block, key block).  Dispatch places workgroup id on
// XCD id % 8, and the workgroups of one XCD share that XCD's L2.
//   mode 0: XCD x takes the key blocks kb = 8j + x, query block fastest, so
//           a key block is read into one L2 only; balanced when the key
//           block count is a multiple of 8.
//   mode 1: XCD x takes the tiles [x*per, (x+1)*per) of the order
//           t = kb*nqb + qb: balanced counts, and an XCD still walks the
//           query blocks of one or two key blocks.
//   mode 2: XCD x takes the query blocks qb = 8j + x of every key block
//           (per = query blocks per XCD): balanced even when the query
//           blocks' extents differ, at the cost of every L2 reading every
//           key block.
struct TileMap {
  int nqb, nkb, mode, per;
};

__device__ __forceinline__ bool tile_of(const TileMap& m, int id, int& qb, int& kb) {
  const int xcd = id & 7, j = id >> 3;
  if (m.mode == 0) {
    qb = j % m.nqb;
    kb = (j / m.nqb) * 8 + xcd;
    return kb < m.nkb;
  }
  if (m.mode == 1) {
    const int t = xcd * m.per + j;
    if (j >= m.per || t >= m.nqb * m.nkb) return false;
    kb = t / m.nqb;
    qb = t % m.nqb;
    return true;
  }
  qb = (j % m.per) * 8 + xcd;
  kb = j / m.per;
  return qb < m.nqb && kb < m.nkb;
}

unsigned grid_of(const TileMap& m) {
  if (m.mode == 0) return (unsigned)(8 * m.nqb * ((m.nkb + 7) / 8));
  if (m.mode == 1) return (unsigned)(8 * m.per);
  return (unsigned)(8 * m.per * m.nkb);
}

TileMap make_tile_map(int nqb, int nkb, int mode) {
  TileMap m{nqb, nkb, mode, 0};
  if (mode == 1) m.per = (int)(((int64_t)nqb * nkb + 7) / 8);
  if (mode == 2) m.per = (nqb + 7) / 8;
  return m;
}

constexpr int kPrefillWaves = 8;
constexpr int kRowsPerWave = 2;
constexpr int kPrefillRows = kPrefillWaves * kRowsPerWave;   // 16 query rows per workgroup

// Work tile = (16 query rows, keys_per_wg keys) of one sequence; each wave
// owns 2 rows and consumes two 16-key tiles per step (the four partials of
// a step are (row, tile) pairs).  Workgroups map to tiles through `map`
// (TileMap: key blocks or query blocks spread over the 8 XCDs).
template <int NHT, bool kFullD>
__global__ void __launch_bounds__(kPrefillWaves * kWave)
indexer_prefill_kernel(IndexerArgs a, int keys_per_wg, TileMap map) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int qb, kb;
  if (!tile_of(map, blockIdx.x, qb, kb)) return;   // block-uniform
  const int b = blockIdx.y;
  const int i0 = qb * kPrefillRows + wave * kRowsPerWave;
  if (i0 >= a.rows) return;
  const int i_last = min(i0 + kRowsPerWave, a.rows) - 1;
  const int pb = row_pos_base(a.pk, b, a.S, a.pos0);
  const int np_last = min(pb + i_last + 1, a.S);
  const int k_begin = kb * keys_per_wg;
  const int k_end = min(k_begin + keys_per_wg, np_last);
  if (k_begin >= k_end) return;

  __shared__ __attribute__((aligned(16))) uint8_t lin_lds[kPrefillWaves * kLinScratch];
  LinLoads<NHT> ll;
  lin_load<NHT>(a, b, i0, i0 + 1, lane, ll);
  v8i qa[kRowsPerWave][kMaxHeadTiles];
  float wq[kRowsPerWave][kMaxHeadTiles][4];
#pragma unroll
  for (int q = 0; q < kRowsPerWave; ++q) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) qa[q][ht] = load_q_tile(a, b, i0 + q, ht, lane);
    load_weights(a, b, i0 + q, lane, 0.5f, wq[q]);
  }
  const LinOp lin = lin_operand<NHT>(ll, wq[0], wq[1], lane, lin_lds + wave * kLinScratch);
  // After the reduce-scatter, lane group g holds row i0 + g/2, tile g%2.
  const int g = lane >> 4;
  const int my_row = i0 + (g >> 1);
  const int my_np = my_row < a.rows ? min(pb + my_row + 1, a.S) : 0;
  float* my_out = a.scores + ((int64_t)b * a.sc_rows_b + min(my_row, a.rows - 1)) * a.ld;
  const v8i* qp[4] = {qa[0], qa[0], qa[1], qa[1]};
  const float(*wp[4])[4] = {wq[0], wq[0], wq[1], wq[1]};

  KeyStream<kFullD> ksr;
  ksr.init(a, b, lane, k_begin);
  const int kl = lane & 15;
  v8i kt0 = ksr.load(k_begin, kl);
  v8i kt1 = ksr.load(k_begin + 16, kl);
  for (int s0 = k_begin; s0 < k_end; s0 += 32) {
    const int s = s0 + 16 * (g & 1) + kl;   // key this lane's result belongs to
    const float ks = ksr.scale(s0, 16 * (g & 1) + kl);
    // next step's tiles (past the block: harmless extra loads)
    const v8i n0 = ksr.load(s0 + 32, kl);
    const v8i n1 = ksr.load(s0 + 48, kl);
    const v8i* kp[4] = {&kt0, &kt1, &kt0, &kt1};
    float p[4];
    tile_partials<NHT>(qp, wp, kp, lin, p);
    const float tot = reduce_scatter4(p[0], p[1], p[2], p[3]);
    if (s < my_np && s < k_end) my_out[s] = tot * ks;
    kt0 = n0;
    kt1 = n1;
  }
}

// Same work tile for d_I = 128, with the key block streamed through LDS in
// sub-blocks of 256 keys (32 KB + 1 KB of scales).  Two buffers are filled
// by global_load_lds DMA a whole sub-block ahead, so each key tile is read
// from memory once per workgroup and the loads are long done when needed.
// Key k of a sub-block occupies 128 bytes; its 16-byte piece p is stored at
// position p ^ f(k), f(k) = (k % 8) ^ ((k / 8) % 2): any 8 consecutive keys
// then hit 8 distinct 16-byte bank groups, and any 16 consecutive keys all
// 64 banks, so the B-operand reads are conflict-free whether the LDS serves
// 8 or 16 lanes of a ds_read_b128 per cycle.
//
// The B operands of step st+1 are read from LDS while step st's MFMAs run
// (two register sets alternate with the step parity).  The per-score
// arithmetic is tile_partials', as in the register-streaming prefill
// kernel.  NW = 4 waves per workgroup lets two workgroups share a CU, so
// one's barrier waits and prologue are covered by the other's work, and
// the two waves on a SIMD alternate between MFMA and VALU phases.
//
constexpr int kSubKeys = 256;
constexpr int kSubBytes = kSubKeys * 128;
constexpr int kLdsWaves = 4;
constexpr int kLdsRows = kLdsWaves * kRowsPerWave;   // 8 query rows per workgroup

// At least 2 waves per SIMD: caps the registers at 256 per lane, which also
// keeps the MFMA results in VGPRs where the epilogue reads them directly.
template <int NHT, int NW>
__global__ void __launch_bounds__(NW * kWave, 2)
indexer_prefill_lds_kernel(IndexerArgs a, int keys_per_wg, TileMap map) {
  constexpr int kRows = NW * kRowsPerWave;
  static_assert(32 % NW == 0 && NW >= 4, "DMA split");
  // Two separate arrays (not one indexed array), so that the compiler can
  // tell LDS reads of one buffer from the DMA in flight into the other.
  __shared__ __attribute__((aligned(16))) uint8_t kbuf0[kSubBytes];
  __shared__ __attribute__((aligned(16))) uint8_t kbuf1[kSubBytes];
  __shared__ __attribute__((aligned(16))) float sbuf0[kSubKeys];
  __shared__ __attribute__((aligned(16))) float sbuf1[kSubKeys];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: keeps the store descriptor scalar
  int qb, kb;
  if (!tile_of(map, blockIdx.x, qb, kb)) return;   // block-uniform
  const int b = blockIdx.y;
  const int i0 = qb * kRows + wave * kRowsPerWave;
  // Block-uniform extent: every wave takes part in the DMA and barriers.
  if (qb * kRows >= a.rows) return;
  const int blk_last = min(qb * kRows + kRows, a.rows) - 1;
  const int k_begin = kb * keys_per_wg;
  const int pb = row_pos_base(a.pk, b, a.S, a.pos0);
  const int k_end = min(k_begin + keys_per_wg, min(pb + blk_last + 1, a.S));
  if (k_begin >= k_end) return;
  const int nsteps = (k_end - k_begin + 31) / 32;   // 32 keys per step, 8 steps per sub-block
  const int nsub = (nsteps + 7) / 8;

  const uint8_t* kseq = a.k_idx + (int64_t)b * a.S * 128;
  const float* sseq = a.k_scale + (int64_t)b * a.S;
  // DMA of sub-block j: wave w issues the 1 KB runs NW*u + w (8 keys each);
  // waves 0..3 also copy 64 key scales each.
  auto dma = [&](int j, uint8_t* kdst, float* sdst) {
    const int key0 = k_begin + j * kSubKeys;
#pragma unroll
    for (int u = 0; u < 32 / NW; ++u) {
      const int inst = u * NW + wave;
      const int kl = inst * 8 + (lane >> 3);   // key within the sub-block
      const int ppos = lane & 7;               // stored piece position
      const int key = min(key0 + kl, a.S - 1);
      const uint8_t* src = kseq + (int64_t)key * 128 + 16 * (ppos ^ ((kl & 7) ^ ((kl >> 3) & 1)));
      dma_x4(src, lds_addr(kdst + inst * 1024));
    }
    if (wave < 4) {
      const int skey = min(key0 + 64 * wave + lane, a.S - 1);
      dma_x1(sseq + skey, lds_addr(sdst + 64 * wave));
    }
  };
  dma(0, kbuf0, sbuf0);

  LinLoads<NHT> ll;
  lin_load<NHT>(a, b, i0, i0 + 1, lane, ll);
  v8i qa[kRowsPerWave][kMaxHeadTiles];
  float wq[kRowsPerWave][kMaxHeadTiles][4];
#pragma unroll
  for (int q = 0; q < kRowsPerWave; ++q) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) qa[q][ht] = load_q_tile(a, b, i0 + q, ht, lane);
    load_weights(a, b, i0 + q, lane, 0.5f, wq[q]);
  }
  // The level operand is built in buffer 1, which no DMA writes before the
  // barrier that publishes sub-block 0.
  static_assert(kLdsWaves * kLinScratch <= kSubBytes, "level scratch");
  const LinOp lin = lin_operand<NHT>(ll, wq[0], wq[1], lane, kbuf1 + wave * kLinScratch);
  // After the reduce-scatter, lane group g holds row i0 + g/2, key tile g%2.
  const int g = lane >> 4;
  const int kl16 = lane & 15;
  const int my_row = i0 + (g >> 1);
  const int my_np = min(my_row < a.rows ? min(pb + my_row + 1, a.S) : 0, k_end);
  // Scores go out through a raw buffer store whose range covers this wave's
  // rows: a lane with nothing to store uses an offset past the range, which
  // the hardware drops, so the step loop has no divergent branch.
  // A wave whose rows all lie past the end (ragged last workgroup) gets an
  // empty range.  The launcher guarantees 2*ld + S fits the 31-bit offsets.
  const int64_t wave_row0 = (int64_t)b * a.sc_rows_b + min(i0, a.rows - 1);
  const int nrows_w = max(0, min(kRowsPerWave, a.rows - i0));
  const int range = nrows_w > 0 ? (int)((int64_t)(nrows_w - 1) * a.ld * 4 + (int64_t)a.S * 4) : 0;
  const __amdgpu_buffer_rsrc_t out_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(a.scores + wave_row0 * a.ld, 0, range, 0x00020000);
  const int lane_row_off = (my_row - i0) * (int)a.ld * 4;
  const v8i* qp[4] = {qa[0], qa[0], qa[1], qa[1]};
  const float(*wp[4])[4] = {wq[0], wq[0], wq[1], wq[1]};

  // B operands of a step (tiles 2*sst and 2*sst+1 of a staged sub-block)
  // and the scale of the key this lane's result of the step belongs to.
  auto read_step = [&](const uint8_t* kbf, const float* sbf, int sst, v8i& t0, v8i& t1, float& ks) {
    const int k0 = 32 * sst + kl16;
    const int k1 = k0 + 16;
    const int f0 = (k0 & 7) ^ ((k0 >> 3) & 1), f1 = (k1 & 7) ^ ((k1 >> 3) & 1);
    const u32x4 a0 = *(const u32x4*)(kbf + k0 * 128 + 16 * ((2 * g) ^ f0));
    const u32x4 a1 = *(const u32x4*)(kbf + k0 * 128 + 16 * ((2 * g + 1) ^ f0));
    const u32x4 b0 = *(const u32x4*)(kbf + k1 * 128 + 16 * ((2 * g) ^ f1));
    const u32x4 b1 = *(const u32x4*)(kbf + k1 * 128 + 16 * ((2 * g + 1) ^ f1));
    t0 = (v8i){(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    t1 = (v8i){(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    ks = sbf[32 * sst + 16 * (g & 1) + kl16];
  };

  // One step: the MFMAs and epilogue of step st with operands (kt0, kt1,
  // ks) while the operands of step st+1 are read from (nk, ns) at
  // sub-block step nsst into (nt0, nt1, nks).  The score and its store
  // offset are returned; put() stores them.
  auto body = [&](int st, const v8i& kt0, const v8i& kt1, float ks, const uint8_t* nk, const float* ns, int nsst,
                  v8i& nt0, v8i& nt1, float& nks, float& val, int& off) {
    read_step(nk, ns, nsst, nt0, nt1, nks);
    const v8i* kp[4] = {&kt0, &kt1, &kt0, &kt1};
    float p[4];
    tile_partials<NHT>(qp, wp, kp, lin, p);
    val = reduce_scatter4(p[0], p[1], p[2], p[3]) * ks;
    const int s = k_begin + 32 * st + 16 * (g & 1) + kl16;
    off = s < my_np ? lane_row_off + s * 4 : INT_MAX;
  };
  auto put = [&](float val, int off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), out_rsrc, off, 0, 0);
  };
  // The 8 steps of sub-block j from buffer (ck, cs); the last one reads the
  // first operands of sub-block j+1 from (ok, os) after the barrier that
  // publishes it, and then sub-block j+2 is sent into (ck, cs).  Register
  // sets A/B alternate with the step parity (sub-blocks start even).
  v8i ktA0, ktA1, ktB0, ktB1;
  float ksA, ksB;
  auto sub_block = [&](int j, uint8_t* ck, float* cs, uint8_t* ok, float* os) {
    const int st0 = 8 * j;
    float val;
    int off;
#pragma unroll
    for (int sst = 0; sst < 8; sst += 2) {
      if (st0 + sst >= nsteps) return;
      if (sst == 6) {
        body(st0 + 6, ktA0, ktA1, ksA, ck, cs, 7, ktB0, ktB1, ksB, val, off);
        if (st0 + 7 >= nsteps) {
          put(val, off);
          return;
        }
        // The DMA wait also waits for this wave's score stores (they count
        // in the same counter), so step 6's store goes out after it: the
        // wait then covers only stores a step or more old, not a fresh one.
        wait_dma();
        put(val, off);
        __syncthreads();   // sub-block j+1 staged; everyone is done reading buffer (ck, cs)
        if (j + 2 < nsub) dma(j + 2, ck, cs);
        body(st0 + 7, ktB0, ktB1, ksB, ok, os, 0, ktA0, ktA1, ksA, val, off);
        put(val, off);
      } else {
        body(st0 + sst, ktA0, ktA1, ksA, ck, cs, sst + 1, ktB0, ktB1, ksB, val, off);
        put(val, off);
        if (st0 + sst + 1 >= nsteps) return;
        body(st0 + sst + 1, ktB0, ktB1, ksB, ck, cs, sst + 2, ktA0, ktA1, ksA, val, off);
        put(val, off);
      }
    }
  };

  // Consume the q and weight loads here, so that the compiler's waits for
  // them do not end up behind (and wait for) the next DMA.
#pragma unroll
  for (int q = 0; q < kRowsPerWave; ++q)
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      asm volatile("" ::"v"(qa[q][ht]));
      asm volatile("" ::"v"(wq[q][ht][0]), "v"(wq[q][ht][1]), "v"(wq[q][ht][2]), "v"(wq[q][ht][3]));
    }
  // ... and the level operand's LDS reads, which must land before buffer 1
  // is reused
  asm volatile("" ::"v"(lin.a), "v"(lin.sc));
  wait_dma();
  __syncthreads();   // sub-block 0 staged
  if (nsub > 1) dma(1, kbuf1, sbuf1);
  read_step(kbuf0, sbuf0, 0, ktA0, ktA1, ksA);
  for (int j = 0; j < nsub; j += 2) {
    sub_block(j, kbuf0, sbuf0, kbuf1, sbuf1);
    if (j + 1 >= nsub) break;
    sub_block(j + 1, kbuf1, sbuf1, kbuf0, sbuf0);
  }
  wait_dma();   // nothing may still write this workgroup's LDS after it ends
}

constexpr int kDecodeWaves = 4;
// Keys per wave of the decode form.  With 3 waves per SIMD (156 VGPRs) the
// GPU holds 3072 waves at once, and a 64-sequence 128K step has 32768 waves
// of 256 keys (10.7 rounds); shorter ranges leave a smaller tail in the last
// round.  Per 64 x 128K decode step: 343, 339, 326 and 323 us for 2048,
// 1024, 512 and 256 keys per wave.
constexpr int kDecodeKeysPerWave = 256;

template <int NHT, bool kFullD>
__global__ void __launch_bounds__(kDecodeWaves * kWave)
indexer_decode_kernel(IndexerArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i = blockIdx.y;
  const int b = blockIdx.z;
  const int np = min(row_pos_base(a.pk, b, a.S, a.pos0) + i + 1, a.S);
  const int k_begin = (blockIdx.x * kDecodeWaves + wave) * kDecodeKeysPerWave;
  if (k_begin >= np) return;
  const int k_end = min(k_begin + kDecodeKeysPerWave, np);

  v8i qa[kMaxHeadTiles];
  float wq[kMaxHeadTiles][4];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) qa[ht] = load_q_tile(a, b, i, ht, lane);
  load_weights(a, b, i, lane, 1.f, wq);
  float* out = a.scores + ((int64_t)b * a.sc_rows_b + i) * a.ld;
  KeyStream<kFullD> ksr;
  ksr.init(a, b, lane, k_begin);
  const int kl = lane & 15;
  v8i kt[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) kt[u] = ksr.load(k_begin + 16 * u, kl);
  for (int s0 = k_begin; s0 < k_end; s0 += 64) {
    const int s = s0 + lane;   // key whose score this lane ends up holding
    const float ks = ksr.scale(s0, lane);
    // The next step's keys are loaded ahead.  The last step reloads its own
    // keys (still in cache) instead: the keys after this wave's range belong
    // to another wave, usually one long finished on another XCD, so reading
    // them again went to HBM (one step in eight, 12% of the stream).
    const int nbase = s0 + 64 < k_end ? s0 + 64 : s0;
    v8i nx[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) nx[u] = ksr.load(nbase + 16 * u, kl);
    const v8i* kp[4] = {&kt[0], &kt[1], &kt[2], &kt[3]};
    float p[4];
    tile_partials_relu<NHT>(qa, wq, kp, p);
    const float tot = reduce_scatter4(p[0], p[1], p[2], p[3]);
    if (s < k_end) out[s] = tot * ks;
#pragma unroll
    for (int u = 0; u < 4; ++u) kt[u] = nx[u];
  }
}

// The LDS-staged kernel stores through 31-bit byte offsets within two rows.
bool lds_path_ok(const IndexerArgs& a) { return (2 * a.ld + (int64_t)a.S) * 4 < (int64_t)INT_MAX; }

// Workgroups of the LDS kernel that are resident at once: two per CU.
int lds_slots() {
  static DeviceOnce cus;
  return 2 * device_once(cus, 256, [](int dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    return n;
  });
}

// Key-block length of the LDS kernel.  A workgroup costs a fixed set-up
// (q tiles, level operand, first key DMA: about kSetupSteps steps of 32
// keys, measured) plus one step per 32 keys, and the launch runs in rounds
// of `slots` workgroups; dispatch takes full key blocks first and each
// query block's shorter last block at the end.  The length (a multiple of
// the 256-key sub-block, up to 16384) minimises an estimate of the
// makespan: whole rounds of full blocks, a last partial round, and the
// short blocks, which after whole rounds mostly start in the slots freed
// by the earliest finishers (kAbsorb: the share of their length that
// still shows).  On 256-row chunks of a 128K prefill this picked the
// fastest of the lengths measured at every position tried; on 512-row
// chunks, allowing 16384 instead of 8192 took a whole 128K indexer pass
// from 56.8 to 56.1 ms (32768 gained nothing more).  The estimate
// assumes query blocks of about equal extent; spans whose extents differ
// by 2048 keys or more (a whole causal triangle) return 0, and the caller
// falls back to its default.  Scores do not depend on it.
int lds_keys_per_wg(const IndexerArgs& a, int nqb, int slots) {
  constexpr double kSetupSteps = 13.0, kAbsorb = 0.3;
  if (!a.pk.seq_lens) {
    const int64_t np_first = min((int64_t)a.pos0 + min(kLdsRows, a.rows), (int64_t)a.S);
    const int64_t np_last = min((int64_t)a.pos0 + a.rows, (int64_t)a.S);
    if (np_last - np_first >= 2048) return 0;
  }
  double best_t = 1e300;
  int best = 2048;
  for (int kpw = 256; kpw <= 16384; kpw += 256) {
    int64_t nfull = 0, npart = 0;
    int dpart = 0;
    for (int qb = 0; qb < nqb; ++qb) {
      const int64_t np = a.pk.seq_lens ? a.S : min((int64_t)a.pos0 + min((qb + 1) * kLdsRows, a.rows), (int64_t)a.S);
      nfull += np / kpw;
      if (np % kpw) {
        ++npart;
        dpart = max(dpart, (int)((np % kpw + 31) / 32));
      }
    }
    nfull *= a.B;
    npart *= a.B;
    const double df = kSetupSteps + kpw / 32, dp = kSetupSteps + dpart;
    const int64_t rounds = nfull / slots, left = nfull % slots, free = slots - left;
    double t = rounds * df + (left ? df : 0.0);
    if (npart) {
      if (left) t += npart <= free ? max(0.0, dp - df) : 0.0;
      else t += kAbsorb * dp;
      if (npart > free) t += dp * (double)((npart - free + slots - 1) / slots);
    }
    if (t < best_t) {
      best_t = t;
      best = kpw;
    }
  }
  return best;
}

// Tile-to-XCD mapping of a prefill launch (see TileMap).  Mode 0 keeps each
// key block in one L2, but with fewer than 8 key blocks it leaves XCDs
// without work, and with query blocks of unequal extent (a causal triangle)
// the XCDs that hold the high key blocks idle.  Mode 2 is balanced in both
// cases: a 4096-row triangle took 95 us with it against 372 us with mode 0,
// while on 256-row chunks of a 128K prefill the two were within noise.
int tile_map_mode(const IndexerArgs& a, int rows_per_wg, int nkb) {
  if (nkb < 8) return 2;
  if (!a.pk.seq_lens) {
    const int64_t np_first = min((int64_t)a.pos0 + min(rows_per_wg, a.rows), (int64_t)a.S);
    const int64_t np_last = min((int64_t)a.pos0 + a.rows, (int64_t)a.S);
    if (np_last - np_first >= 2048) return 2;
  }
  return 0;
}

template <int NHT, bool kFullD>
hipError_t launch_nht(const IndexerArgs& a, bool decode_form, hipStream_t st) {
  // longest row (with per-sequence lengths the host only knows the bound S)
  const int np_max = a.pk.seq_lens ? a.S : min(a.pos0 + a.rows, a.S);
  const bool lds_ok = kFullD && !a.pk.page_table && lds_path_ok(a);
  if (decode_form) {
    const int per_wg = kDecodeWaves * kDecodeKeysPerWave;
    dim3 grid((np_max + per_wg - 1) / per_wg, a.rows, a.B);
    hipLaunchKernelGGL((indexer_decode_kernel<NHT, kFullD>), grid, dim3(kDecodeWaves * kWave), 0, st, a);
  } else {
    const int rows_per_wg = lds_ok ? kLdsRows : kPrefillRows;
    const int nqb = (a.rows + rows_per_wg - 1) / rows_per_wg;
    // Key-block length: the LDS kernel's makespan estimate where it
    // applies; otherwise 2048 keys (amortising the q loads, 8 KB per row),
    // halved while that leaves fewer than ~512 workgroups.  Results do not
    // depend on it.
    int keys = lds_ok ? lds_keys_per_wg(a, nqb, lds_slots()) : 0;
    if (keys == 0) {
      keys = 2048;
      while (keys > 256) {
        const long long kblocks = (np_max + keys - 1) / keys;
        if ((long long)nqb * kblocks * a.B >= 512) break;
        keys >>= 1;
      }
    }
    const int nkb = (np_max + keys - 1) / keys;
    const TileMap map = make_tile_map(nqb, nkb, tile_map_mode(a, rows_per_wg, nkb));
    dim3 grid(grid_of(map), a.B);
    if (lds_ok)
      hipLaunchKernelGGL((indexer_prefill_lds_kernel<NHT, kLdsWaves>), grid, dim3(kLdsWaves * kWave), 0, st, a, keys, map);
    else
      hipLaunchKernelGGL((indexer_prefill_kernel<NHT, kFullD>), grid, dim3(kPrefillWaves * kWave), 0, st, a, keys, map);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, bool decode_form, hipStream_t st) {
  if (a.rows <= 0 || a.B <= 0) return hipSuccess;
  if (a.dI == 128) {
    switch ((a.HI + 15) >> 4) {
      case 1: return launch_nht<1, true>(a, decode_form, st);
      case 2: return launch_nht<2, true>(a, decode_form, st);
      case 3: return launch_nht<3, true>(a, decode_form, st);
      default: return launch_nht<4, true>(a, decode_form, st);
    }
  }
  switch ((a.HI + 15) >> 4) {
    case 1: return launch_nht<1, false>(a, decode_form, st);
    case 2: return launch_nht<2, false>(a, decode_form, st);
    case 3: return launch_nht<3, false>(a, decode_form, st);
    default: return launch_nht<4, false>(a, decode_form, st);
  }
}

}  // namespace dsa
