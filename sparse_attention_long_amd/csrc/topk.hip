// Per-row top-k selection (page "DeepSeek-V3.2: sparse attention, scaled RL
// and synthetic agent environments": the selected set S_t of Sec. 1.1 /
// Eq. (4); rows shorter than k keep everything, Sec. 5.1; equal scores at
// the cutoff are legitimate, Sec. 5.2 near Eq. (18) -- here they go to the
// lower index).
//
// One workgroup per row.  Scores are mapped to order-preserving 32-bit keys
// (NaN lowest, -0 == +0) and the m-th largest key tau is found by a radix
// select with 11/11/10-bit digits:
//   pass 1 (HBM): LDS histogram of the top 11 bits -> bin b1 holding tau;
//   pass 2 (HBM or cache): keys above bin b1 are marked in an LDS bitmap,
//          keys inside bin b1 are compacted into an LDS candidate list;
//   digits 2 and 3 are resolved on the candidates in LDS.
// (If bin b1 holds more keys than the candidate list can, digits 2 and 3
// take two more passes over the row instead.)  Keys above tau go into the
// bitmap, keys equal to tau into a tie bitmap; the first (m - #above) ties
// in index order are kept and the bitmap is emitted in ascending order with
// a block-wide popcount prefix sum.  The row is read at most twice in the
// common case; the selection needs no sort.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kCandCap = 4096;
constexpr int kMaxKV = 262144;
constexpr int kBins1 = 2048;   // bits 31..21
constexpr int kBins2 = 2048;   // bits 20..10
constexpr int kBins3 = 1024;   // bits 9..0

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (x != x) return 0u;                    // NaN below everything
  if (u == 0x80000000u) u = 0u;             // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct Shared {
  uint32_t scan[kWaves];
  uint32_t bin, above, ncand;
};

// Exclusive prefix sum over the block in thread order.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, Shared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) sh.scan[wave] = x;
  __syncthreads();
  uint32_t pre = 0;
  for (int w = 0; w < wave; ++w) pre += sh.scan[w];
  __syncthreads();
  return pre + x - v;
}

// Find bin b with (count of keys in bins > b) < rank <= (count in bins >= b),
// scanning from the top bin.  rank is 1-based.  Result in sh.bin / sh.above.
__device__ void find_bin(const uint32_t* hist, int nbins, uint32_t rank, Shared& sh) {
  const int per = nbins / kThreads;
  const int top = nbins - 1 - (int)threadIdx.x * per;
  uint32_t local = 0;
  for (int j = 0; j < per; ++j) local += hist[top - j];
  const uint32_t excl = block_exclusive_scan(local, sh);
  if (excl < rank && rank <= excl + local) {
    uint32_t cum = excl;
    for (int j = 0; j < per; ++j) {
      const uint32_t c = hist[top - j];
      if (cum + c >= rank) { sh.bin = (uint32_t)(top - j); sh.above = cum; break; }
      cum += c;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void set_bit(uint32_t* bm, int e) { atomicOr(&bm[e >> 5], 1u << (e & 31)); }

// Keep only the lowest `keep` set bits of w.
__device__ __forceinline__ uint32_t keep_lowest(uint32_t w, uint32_t keep) {
  uint32_t r = 0;
  while (keep-- > 0 && w) { const uint32_t low = w & (0u - w); r |= low; w ^= low; }
  return r;
}

__global__ void __launch_bounds__(kThreads) topk_kernel(TopkArgs a) {
  extern __shared__ uint32_t lds[];
  __shared__ Shared sh;
  const int t = threadIdx.x;
  const int b = blockIdx.x / a.rows;
  const int i = blockIdx.x % a.rows;
  const int n = min(a.pos0 + i + 1, a.S);
  const int m = min(a.k, n);
  int32_t* out = a.idx + ((int64_t)b * a.idx_rows_b + i) * a.k;
  if (n <= a.k) {   // short row: every candidate is selected
    for (int j = t; j < a.k; j += kThreads) out[j] = j < n ? j : -1;
    return;
  }
  const float* x = a.scores + ((int64_t)b * a.sc_rows_b + i) * a.ld;
  const int nwords = (n + 31) >> 5;
  uint32_t* hist = lds;                          // kBins1 (reused for digits 2, 3)
  uint32_t* selbm = hist + kBins1;               // nwords
  uint32_t* tiebm = selbm + ((a.S + 31) >> 5);   // nwords
  uint32_t* ckey = tiebm + ((a.S + 31) >> 5);    // kCandCap
  uint32_t* cidx = ckey + kCandCap;              // kCandCap

  for (int j = t; j < kBins1; j += kThreads) hist[j] = 0;
  for (int j = t; j < nwords; j += kThreads) { selbm[j] = 0; tiebm[j] = 0; }
  if (t == 0) sh.ncand = 0;
  __syncthreads();

  // ---- pass 1: digit-1 histogram
  for (int e0 = t; e0 < n; e0 += 4 * kThreads) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) { const int e = e0 + u * kThreads; v[u] = e < n ? x[e] : 0.f; }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (e0 + u * kThreads < n) atomicAdd(&hist[order_key(v[u]) >> 21], 1u);
  }
  __syncthreads();
  find_bin(hist, kBins1, (uint32_t)m, sh);
  const uint32_t b1 = sh.bin;
  const uint32_t rank1 = (uint32_t)m - sh.above;   // rank of tau inside bin b1
  const uint32_t c1 = hist[b1];
  __syncthreads();

  uint32_t tau, need;
  if (c1 <= kCandCap) {
    // ---- pass 2: mark keys above bin b1, collect bin b1
    for (int e0 = t; e0 < n; e0 += 4 * kThreads) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) { const int e = e0 + u * kThreads; v[u] = e < n ? x[e] : 0.f; }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * kThreads;
        if (e < n) {
          const uint32_t key = order_key(v[u]);
          const uint32_t d = key >> 21;
          if (d > b1) set_bit(selbm, e);
          else if (d == b1) { const uint32_t pos = atomicAdd(&sh.ncand, 1u); ckey[pos] = key; cidx[pos] = (uint32_t)e; }
        }
      }
    }
    for (int j = t; j < kBins2; j += kThreads) hist[j] = 0;
    __syncthreads();
    const int nc = (int)sh.ncand;
    for (int c = t; c < nc; c += kThreads) atomicAdd(&hist[(ckey[c] >> 10) & 0x7FFu], 1u);
    __syncthreads();
    find_bin(hist, kBins2, rank1, sh);
    const uint32_t b2 = sh.bin;
    const uint32_t rank2 = rank1 - sh.above;
    __syncthreads();
    for (int j = t; j < kBins3; j += kThreads) hist[j] = 0;
    __syncthreads();
    for (int c = t; c < nc; c += kThreads)
      if (((ckey[c] >> 10) & 0x7FFu) == b2) atomicAdd(&hist[ckey[c] & 0x3FFu], 1u);
    __syncthreads();
    find_bin(hist, kBins3, rank2, sh);
    tau = (b1 << 21) | (b2 << 10) | sh.bin;
    need = rank2 - sh.above;
    for (int c = t; c < nc; c += kThreads) {
      const uint32_t key = ckey[c];
      if (key > tau) set_bit(selbm, (int)cidx[c]);
      else if (key == tau) set_bit(tiebm, (int)cidx[c]);
    }
  } else {
    // ---- wide bin: resolve digits 2 and 3 with extra passes over the row
    for (int j = t; j < kBins2; j += kThreads) hist[j] = 0;
    __syncthreads();
    for (int e = t; e < n; e += kThreads) {
      const uint32_t key = order_key(x[e]);
      if ((key >> 21) == b1) atomicAdd(&hist[(key >> 10) & 0x7FFu], 1u);
    }
    __syncthreads();
    find_bin(hist, kBins2, rank1, sh);
    const uint32_t pre = (b1 << 11) | sh.bin;
    const uint32_t rank2 = rank1 - sh.above;
    __syncthreads();
    for (int j = t; j < kBins3; j += kThreads) hist[j] = 0;
    __syncthreads();
    for (int e = t; e < n; e += kThreads) {
      const uint32_t key = order_key(x[e]);
      if ((key >> 10) == pre) atomicAdd(&hist[key & 0x3FFu], 1u);
    }
    __syncthreads();
    find_bin(hist, kBins3, rank2, sh);
    tau = (pre << 10) | sh.bin;
    need = rank2 - sh.above;
    for (int e = t; e < n; e += kThreads) {
      const uint32_t key = order_key(x[e]);
      if (key > tau) set_bit(selbm, e);
      else if (key == tau) set_bit(tiebm, e);
    }
  }
  __syncthreads();

  // ---- emit: keep the first `need` ties, then all marked indices ascending
  const int wpt = (nwords + kThreads - 1) / kThreads;
  const int w0 = min(t * wpt, nwords), w1 = min(w0 + wpt, nwords);
  uint32_t tl = 0;
  for (int w = w0; w < w1; ++w) tl += __popc(tiebm[w]);
  uint32_t tpre = block_exclusive_scan(tl, sh);
  uint32_t sl = 0;
  for (int w = w0; w < w1; ++w) {
    const uint32_t tw = tiebm[w];
    const uint32_t c = __popc(tw);
    uint32_t kept = 0;
    if (tpre < need) kept = (tpre + c <= need) ? tw : keep_lowest(tw, need - tpre);
    tpre += c;
    const uint32_t s = selbm[w] | kept;
    selbm[w] = s;
    sl += __popc(s);
  }
  uint32_t pos = block_exclusive_scan(sl, sh);
  for (int w = w0; w < w1; ++w) {
    uint32_t s = selbm[w];
    while (s) {
      const int bit = __ffs(s) - 1;
      if (pos < (uint32_t)m) out[pos] = (w << 5) + bit;   // exactly m bits are set; guard anyway
      ++pos;
      s &= s - 1;
    }
  }
  for (int j = m + t; j < a.k; j += kThreads) out[j] = -1;
}

}  // namespace

int topk_max_kv() { return kMaxKV; }

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.rows <= 0 || a.B <= 0) return hipSuccess;
  const size_t words = (size_t)((a.S + 31) >> 5);
  const size_t lds = (kBins1 + 2 * words + 2 * kCandCap) * sizeof(uint32_t);
  static bool attr_set = false;
  if (!attr_set) {
    const size_t max_lds = (kBins1 + 2 * (size_t)(kMaxKV / 32) + 2 * kCandCap) * sizeof(uint32_t);
    const hipError_t e = hipFuncSetAttribute((const void*)topk_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)max_lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)(a.B * a.rows)), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace dsa
