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
// Two work shapes share the per-tile arithmetic (so they give bit-identical
// scores):
//  * prefill: a wave keeps the A operands (q) of 4 query rows in registers
//    and streams 16-key tiles; the 4 rows' partials are reduce-scattered so
//    each 16-lane row ends with one query's 16 scores.
//  * decode: a wave keeps one row's q and streams 4 key tiles per step; the
//    reduce-scatter leaves 64 consecutive keys' scores, one per lane.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kMaxHeadTiles = 4;   // H_I <= 64

// A operand: 16 heads x 128 bytes of one query row (zero outside H_I/d_I).
__device__ __forceinline__ v8i load_q_tile(const IndexerArgs& a, int b, int i, int ht, int lane) {
  v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
  const int h = ht * 16 + (lane & 15);
  const int off = 32 * (lane >> 4);
  if (i < a.rows && h < a.HI) {
    const uint8_t* base = a.q_idx + (((int64_t)b * a.qrows_b + i) * a.HI + h) * a.dI + off;
    if (off + 16 <= a.dI) {
      const u32x4 x = *(const u32x4*)base;
      r[0] = x[0]; r[1] = x[1]; r[2] = x[2]; r[3] = x[3];
    }
    if (off + 32 <= a.dI) {
      const u32x4 x = *(const u32x4*)(base + 16);
      r[4] = x[0]; r[5] = x[1]; r[6] = x[2]; r[7] = x[3];
    }
  }
  return r;
}

// B operand: 16 keys x 128 bytes; lane holds key s (zero if s >= S).
__device__ __forceinline__ v8i load_k_tile(const IndexerArgs& a, int b, int s, int lane) {
  v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
  const int off = 32 * (lane >> 4);
  if (s < a.S) {
    const uint8_t* base = a.k_idx + ((int64_t)b * a.S + s) * a.dI + off;
    if (off + 16 <= a.dI) {
      const u32x4 x = *(const u32x4*)base;
      r[0] = x[0]; r[1] = x[1]; r[2] = x[2]; r[3] = x[3];
    }
    if (off + 32 <= a.dI) {
      const u32x4 x = *(const u32x4*)(base + 16);
      r[4] = x[0]; r[5] = x[1]; r[6] = x[2]; r[7] = x[3];
    }
  }
  return r;
}

// Folded head weights w[t,j]*qs[t] for the 4 heads (per head tile) this lane
// sees in the MFMA result: head 16*ht + 4*(lane/16) + r.
__device__ __forceinline__ void load_weights(const IndexerArgs& a, int b, int i, int lane,
                                             float (&wq)[kMaxHeadTiles][4]) {
  const bool row_ok = i < a.rows;
  const int64_t row = (int64_t)b * a.qrows_b + i;
  const float qs = row_ok ? a.q_scale[row] : 0.f;
#pragma unroll
  for (int ht = 0; ht < kMaxHeadTiles; ++ht)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 16 * ht + 4 * (lane >> 4) + r;
      wq[ht][r] = (row_ok && h < a.HI) ? bf16_to_f32(a.w[row * a.HI + h]) * qs : 0.f;
    }
}

// Partial head sum of one query row against one 16-key tile: this lane's
// 16 heads (4 per head tile), sum_h wq[h] * ReLU(dot_h), in a fixed order.
__device__ __forceinline__ float tile_partial(const v8i (&qa)[kMaxHeadTiles], const float (&wq)[kMaxHeadTiles][4],
                                              const v8i& kt, int n_head_tiles) {
  float acc = 0.f;
#pragma unroll
  for (int ht = 0; ht < kMaxHeadTiles; ++ht) {
    if (ht < n_head_tiles) {
      const v4f d = mfma_fp8_16x16x128(qa[ht], kt);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc = fmaf(wq[ht][r], fmaxf(d[r], 0.f), acc);
    }
  }
  return acc;
}

constexpr int kPrefillWaves = 8;
constexpr int kRowsPerWave = 4;
constexpr int kPrefillRows = kPrefillWaves * kRowsPerWave;   // 32 query rows per workgroup

__global__ void __launch_bounds__(kPrefillWaves * kWave)
indexer_prefill_kernel(IndexerArgs a, int keys_per_wg) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.z;
  const int i0 = blockIdx.y * kPrefillRows + wave * kRowsPerWave;
  if (i0 >= a.rows) return;
  const int i_last = min(i0 + kRowsPerWave, a.rows) - 1;
  const int np_last = min(a.pos0 + i_last + 1, a.S);
  const int k_begin = blockIdx.x * keys_per_wg;
  const int k_end = min(k_begin + keys_per_wg, np_last);
  if (k_begin >= k_end) return;
  const int nht = (a.HI + 15) >> 4;

  v8i qa[kRowsPerWave][kMaxHeadTiles];
  float wq[kRowsPerWave][kMaxHeadTiles][4];
#pragma unroll
  for (int q = 0; q < kRowsPerWave; ++q) {
#pragma unroll
    for (int ht = 0; ht < kMaxHeadTiles; ++ht) qa[q][ht] = load_q_tile(a, b, i0 + q, ht, lane);
    load_weights(a, b, i0 + q, lane, wq[q]);
  }
  // This lane stores the scores of query row i0 + lane/16.
  const int my_row = i0 + (lane >> 4);
  const int my_np = my_row < a.rows ? min(a.pos0 + my_row + 1, a.S) : 0;
  float* my_out = a.scores + ((int64_t)b * a.sc_rows_b + min(my_row, a.rows - 1)) * a.ld;

  v8i kt = load_k_tile(a, b, k_begin + (lane & 15), lane);
  for (int s0 = k_begin; s0 < k_end; s0 += 16) {
    const int s = s0 + (lane & 15);
    const float ks = s < a.S ? a.k_scale[(int64_t)b * a.S + s] : 0.f;
    const v8i kt_next = (s0 + 16 < k_end) ? load_k_tile(a, b, s + 16, lane) : kt;
    float p[kRowsPerWave];
#pragma unroll
    for (int q = 0; q < kRowsPerWave; ++q) p[q] = tile_partial(qa[q], wq[q], kt, nht);
    const float tot = reduce_scatter4(p[0], p[1], p[2], p[3]);
    if (s < my_np) my_out[s] = tot * ks;
    kt = kt_next;
  }
}

constexpr int kDecodeWaves = 4;
constexpr int kDecodeKeysPerWave = 512;

__global__ void __launch_bounds__(kDecodeWaves * kWave)
indexer_decode_kernel(IndexerArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i = blockIdx.y;
  const int b = blockIdx.z;
  const int np = min(a.pos0 + i + 1, a.S);
  const int k_begin = (blockIdx.x * kDecodeWaves + wave) * kDecodeKeysPerWave;
  if (k_begin >= np) return;
  const int k_end = min(k_begin + kDecodeKeysPerWave, np);
  const int nht = (a.HI + 15) >> 4;

  v8i qa[kMaxHeadTiles];
  float wq[kMaxHeadTiles][4];
#pragma unroll
  for (int ht = 0; ht < kMaxHeadTiles; ++ht) qa[ht] = load_q_tile(a, b, i, ht, lane);
  load_weights(a, b, i, lane, wq);
  float* out = a.scores + ((int64_t)b * a.sc_rows_b + i) * a.ld;

  v8i kt[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) kt[u] = load_k_tile(a, b, k_begin + 16 * u + (lane & 15), lane);
  for (int s0 = k_begin; s0 < k_end; s0 += 64) {
    const int s = s0 + lane;   // key whose score this lane ends up holding
    const float ks = s < a.S ? a.k_scale[(int64_t)b * a.S + s] : 0.f;
    v8i nx[4];
    const bool more = s0 + 64 < k_end;
#pragma unroll
    for (int u = 0; u < 4; ++u) nx[u] = more ? load_k_tile(a, b, s0 + 64 + 16 * u + (lane & 15), lane) : kt[u];
    float p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) p[u] = tile_partial(qa, wq, kt[u], nht);
    const float tot = reduce_scatter4(p[0], p[1], p[2], p[3]);
    if (s < k_end) out[s] = tot * ks;
#pragma unroll
    for (int u = 0; u < 4; ++u) kt[u] = nx[u];
  }
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, bool decode_form, hipStream_t st) {
  if (a.rows <= 0 || a.B <= 0) return hipSuccess;
  const int np_max = min(a.pos0 + a.rows, a.S);   // longest row
  if (decode_form) {
    const int per_wg = kDecodeWaves * kDecodeKeysPerWave;
    dim3 grid((np_max + per_wg - 1) / per_wg, a.rows, a.B);
    hipLaunchKernelGGL(indexer_decode_kernel, grid, dim3(kDecodeWaves * kWave), 0, st, a);
  } else {
    const int qblocks = (a.rows + kPrefillRows - 1) / kPrefillRows;
    // Larger key blocks amortise the q loads (8 KB per row); smaller ones
    // give enough workgroups for small problems.  Results do not depend on it.
    int keys = 2048;
    while (keys > 256) {
      const long long kblocks = (np_max + keys - 1) / keys;
      if ((long long)qblocks * kblocks * a.B >= 4096) break;
      keys >>= 1;
    }
    dim3 grid((np_max + keys - 1) / keys, qblocks, a.B);
    hipLaunchKernelGGL(indexer_prefill_kernel, grid, dim3(kPrefillWaves * kWave), 0, st, a, keys);
  }
  return hipGetLastError();
}

}  // namespace dsa
