// Opt-in device check of the inputs whose values the host cannot see (the
// analysis page, Sec. 5.1: kernels should check valid lengths and the
// finiteness of scales, since odd scales, NaN and many equal scores
// destabilise the selection).  The stage kernels never fault on such values
// (lengths and page entries are clamped, NaN scores rank last), so this
// check is a separate call whose counts the caller reads when it wants them.
//
// One grid covers four kinds of work, each a contiguous range of workgroups:
// query rows (scales and head weights), cache tokens (key scales), selection
// rows (one wave per row) and sequences (length and page entries).  Every
// thread counts locally; a wave adds its totals to the caller's counters
// with one atomic per non-zero counter.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;

__global__ void zero_counts_kernel(int32_t* counts) {
  if (threadIdx.x < kValidateCounts) counts[threadIdx.x] = 0;
}

// Not (finite and > 0); NaN compares false both ways.
__device__ __forceinline__ bool bad_scale(float x) { return !(x > 0.f && x <= 3.402823466e38f); }
// bf16 with an all-ones exponent: inf or NaN.
__device__ __forceinline__ bool bf16_nonfinite(uint16_t h) { return (h & 0x7F80u) == 0x7F80u; }

__device__ __forceinline__ void wave_add(int32_t* counter, int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  if ((threadIdx.x & 63) == 0 && v != 0) atomicAdd(counter, v);
}

__global__ void __launch_bounds__(kThreads) validate_kernel(ValidateArgs a) {
  const int lane = threadIdx.x & 63;
  int blk = blockIdx.x;
  int c_q = 0, c_w = 0, c_k = 0, c_idx = 0, c_row = 0, c_len = 0, c_page = 0;

  if (blk < a.blocks_q) {
    // query rows: q_scale [B, n_q] and w [B, n_q, HI]
    const int64_t rows = (int64_t)a.B * a.n_q;
    for (int64_t r = (int64_t)blk * kThreads + threadIdx.x; r < rows; r += (int64_t)a.blocks_q * kThreads) {
      if (a.q_scale && bad_scale(a.q_scale[r])) ++c_q;
      if (a.w)
        for (int j = 0; j < a.HI; ++j) c_w += bf16_nonfinite(a.w[r * a.HI + j]) ? 1 : 0;
    }
  } else if ((blk -= a.blocks_q) < a.blocks_k) {
    // cache tokens a query row can see: key scales
    const int64_t toks = (int64_t)a.B * a.S;
    for (int64_t t = (int64_t)blk * kThreads + threadIdx.x; t < toks; t += (int64_t)a.blocks_k * kThreads) {
      const int b = (int)(t / a.S), s = (int)(t % a.S);
      const int len = a.pk.seq_lens ? seq_len_of(a.pk, b, a.S) : min(a.S, a.q_pos0 + a.n_q);
      if (s < len && bad_scale(a.k_scale[cache_row(a.pk, b, a.S, s)])) ++c_k;
    }
  } else if ((blk -= a.blocks_k) < a.blocks_idx) {
    // selection rows, one wave each: entries outside {-1} U [0, n_p), and
    // rows whose valid entries are not strictly ascending or not followed
    // by -1 padding only
    const int64_t rows = (int64_t)a.B * a.n_q;
    const int64_t r = (int64_t)blk * (kThreads / kWave) + (threadIdx.x >> 6);
    if (r < rows) {
      const int b = (int)(r / a.n_q), i = (int)(r % a.n_q);
      const int len = seq_len_of(a.pk, b, a.S);
      const int n = min(row_pos_base(a.pk, b, a.S, a.q_pos0) + i + 1, len);
      const int32_t* row = a.idx + r * a.k;
      int prev_last = -1;       // last entry of the previous 64 (lane 63's)
      bool padded = false;      // a -1 was seen before this group
      bool noncanon = false;
      for (int j0 = 0; j0 < a.k; j0 += kWave) {
        const int j = j0 + lane;
        const int v = j < a.k ? row[j] : -1;
        if (j < a.k && v != -1 && (v < 0 || v >= n)) ++c_idx;
        int prev = __shfl_up(v, 1, kWave);
        if (lane == 0) prev = prev_last;
        const bool first = j == 0;
        const bool pad_before = padded || (!first && prev == -1);
        if (j < a.k && v != -1 && ((!first && pad_before) || (!first && prev != -1 && v <= prev))) noncanon = true;
        const uint64_t pads = __ballot(j < a.k && v == -1);
        padded = padded || pads != 0;
        prev_last = __shfl(v, 63, kWave);
      }
      c_row = __ballot(noncanon) != 0 && lane == 0 ? 1 : 0;
    }
  } else if ((blk -= a.blocks_idx) < a.blocks_seq) {
    // sequences of a variable-length layout: lengths and page entries
    for (int b = blk * kThreads + threadIdx.x; b < a.B; b += a.blocks_seq * kThreads) {
      const int raw = a.pk.seq_lens[b];
      if (raw < a.n_q || raw > a.S) ++c_len;
      if (a.pk.page_table) {
        const int used = (seq_len_of(a.pk, b, a.S) + a.pk.page_size - 1) / a.pk.page_size;
        for (int j = 0; j < used; ++j) {
          const int e = a.pk.page_table[(int64_t)b * a.pk.max_pages + j];
          if (e < 0 || e >= a.pk.num_pages) ++c_page;
        }
      }
    }
  }
  wave_add(&a.counts[0], c_q);
  wave_add(&a.counts[1], c_w);
  wave_add(&a.counts[2], c_k);
  wave_add(&a.counts[3], c_idx);
  wave_add(&a.counts[4], c_row);
  wave_add(&a.counts[5], c_len);
  wave_add(&a.counts[6], c_page);
}

}  // namespace

hipError_t launch_validate(ValidateArgs a, hipStream_t st) {
  hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(64), 0, st, a.counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)a.B * a.n_q;
  const int64_t toks = (int64_t)a.B * a.S;
  auto blocks = [](int64_t n, int64_t per) { return (int)std::min<int64_t>((n + per - 1) / per, 2048); };
  a.blocks_q = (a.q_scale || a.w) ? blocks(rows, kThreads) : 0;
  a.blocks_k = a.k_scale ? blocks(toks, kThreads) : 0;
  a.blocks_idx = a.idx ? (int)((rows + kThreads / kWave - 1) / (kThreads / kWave)) : 0;
  a.blocks_seq = a.pk.seq_lens ? blocks(a.B, kThreads) : 0;
  const int64_t grid = (int64_t)a.blocks_q + a.blocks_k + a.blocks_idx + a.blocks_seq;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(validate_kernel, dim3((unsigned)grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa
