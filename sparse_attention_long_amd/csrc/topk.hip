// Per-row top-k selection (page "DeepSeek-V3.2: sparse attention, scaled RL
// and synthetic agent environments": the selected set S_t of Sec. 1.1 /
// Eq. (4); rows shorter than k keep everything, Sec. 5.1; equal scores at
// the cutoff are legitimate, Sec. 5.2 near Eq. (18) -- here they go to the
// lower index).
//
// One workgroup of 1024 threads per row.  Scores are mapped to
// order-preserving 32-bit keys (NaN lowest, -0 == +0); tau, the m-th largest
// key, is found as follows.
//   Sampled single pass (the usual path): 2048 scores (32 blocks of 64
//          spread over the row) give a provisional cutoff lo, the lower
//          edge of the 13-bit bin (sign, exponent, 4 mantissa bits) that
//          holds the sample's rank-r key, with r set so that about 2m keys
//          of the row are expected at or above lo.  One pass over the row
//          appends every key >= lo, with its index, to an LDS candidate list
//          (one LDS atomic per wave per iteration; ballots give the slots).
//          If between m and `cap` keys were collected, tau is among them:
//          its 13-bit bin, then the 10- and 9-bit digits, are resolved on
//          the candidates in LDS.
//   Fallback (the sample missed): pass 1 builds the LDS histogram of the
//          13-bit digit over the whole row and fixes tau's bin b1; pass 2
//          marks the keys above b1 and collects bin b1 into the candidate
//          list; a bin wider than the list takes one more pass per digit.
// Keys above tau go into a selection bitmap and keys equal to tau into a
// tie bitmap; the first (m - #above) ties in index order are kept, and the
// bitmap is emitted in ascending order with a block-wide popcount prefix
// sum.  The selection needs no sort.
//
// The row is streamed with 16-byte loads, four per thread in flight (64 KB
// per workgroup), after a scalar head that reaches 16-byte alignment.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxKV = 262144;
constexpr int kShift1 = 19;                 // digit 1 = key bits 31..19
constexpr int kBins1 = 1 << (32 - kShift1); // 8192
constexpr int kShift2 = 9;                  // digit 2 = key bits 18..9
constexpr int kBins2 = 1 << (kShift1 - kShift2);   // 1024
constexpr int kBins3 = 1 << kShift2;        // digit 3 = key bits 8..0: 512
constexpr int kMaxCand = 8192;
constexpr int kDynLds = 163840 - 1024;      // dynamic LDS bytes (the rest: static)
constexpr int kUnroll = 4;                  // 16-byte loads in flight per thread

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
// scanning from the top bin.  rank is 1-based and at most the total count.
// Thread t owns bins top_t, top_t - 1, ... (per of them); the scan in thread
// order is then a scan from the top bin down.  Result in sh.bin / sh.above.
__device__ void find_bin(const uint32_t* hist, int nbins, uint32_t rank, Shared& sh) {
  const int per = (nbins + kThreads - 1) / kThreads;
  const int top = nbins - 1 - (int)threadIdx.x * per;
  uint32_t local = 0;
  for (int j = 0; j < per; ++j)
    if (top - j >= 0) local += hist[top - j];
  const uint32_t excl = block_exclusive_scan(local, sh);
  if (local > 0 && excl < rank && rank <= excl + local) {
    uint32_t cum = excl;
    for (int j = 0; j < per && top - j >= 0; ++j) {
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

// Append (key, e) for the lanes with c set: one LDS atomic per wave.  Must be
// reached by whole waves (wave-uniform control flow).
__device__ __forceinline__ void append_wave(bool c, uint32_t key, uint32_t e, uint32_t* ckey, uint32_t* cidx,
                                            int cap, Shared& sh) {
  const uint64_t m = __ballot(c);
  if (m == 0) return;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)m) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(&sh.ncand, (uint32_t)__popcll(m));
  base = __shfl(base, leader, 64);
  if (c) {
    const uint64_t below = lane == 0 ? 0ull : (m & (~0ull >> (64 - lane)));
    const uint32_t pos = base + (uint32_t)__popcll(below);
    if (pos < (uint32_t)cap) { ckey[pos] = key; cidx[pos] = e; }
  }
}

// Exclusive prefix over the wave of per-lane counts below 32, and the
// wave total, from five ballots (no LDS traffic).
__device__ __forceinline__ uint32_t wave_prefix_small(uint32_t cnt, uint32_t& total) {
  uint32_t pre = 0;
  total = 0;
#pragma unroll
  for (int bit = 0; bit < 5; ++bit) {
    const uint64_t bm = __ballot((cnt >> bit) & 1u);
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
    pre += below << bit;
    total += (uint32_t)__popcll(bm) << bit;
  }
  return pre;
}

// The row split for vector loads: elements [0, h) are read one by one
// (h < 4 reaches 16-byte alignment), then nq float4s, then a tail of < 4.
struct RowSplit {
  const float* x;
  const float4* xv;
  int n, h, nq, tail0;
  __device__ __forceinline__ RowSplit(const float* p, int n_) : x(p), n(n_) {
    const int mis = (int)(((uintptr_t)p >> 2) & 3);
    h = min(n, (4 - mis) & 3);
    nq = (n - h) >> 2;
    tail0 = h + 4 * nq;
    xv = (const float4*)(p + h);
  }
};

// Calls f(e, key, valid) for every element of the row.  The vector part runs
// the same number of iterations in every thread (block-uniform), so f may
// use wave-wide operations; elements past the end come with valid = false.
// The < 8 head and tail elements are visited by threads 0..7 afterwards with
// a per-thread (not wave-uniform) call g(e, key).
template <class F, class G>
__device__ __forceinline__ void scan_row(const RowSplit& r, F&& f, G&& g) {
  const int t = threadIdx.x;
  const int iters = (r.nq + kThreads * kUnroll - 1) / (kThreads * kUnroll);
  for (int it = 0; it < iters; ++it) {
    float4 v[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int q = (it * kUnroll + u) * kThreads + t;
      ok[u] = q < r.nq;
      v[u] = r.xv[ok[u] ? q : 0];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e = r.h + 4 * ((it * kUnroll + u) * kThreads + t);
      f(e + 0, order_key(v[u].x), ok[u]);
      f(e + 1, order_key(v[u].y), ok[u]);
      f(e + 2, order_key(v[u].z), ok[u]);
      f(e + 3, order_key(v[u].w), ok[u]);
    }
  }
  if (t < r.h) g(t, order_key(r.x[t]));
  if (t >= 4 && t - 4 < r.n - r.tail0) g(r.tail0 + t - 4, order_key(r.x[r.tail0 + t - 4]));
}

// Candidates of a row collected by the parts of topk_collect_kernel.
struct Parts {
  uint32_t* cnt;   // [rows_total * nparts] keys each part found at or above its cutoff
  uint32_t* key;   // [rows_total * nparts * kCapPart]
  uint32_t* idx;
  int nparts;
};
constexpr int kCapPart = 4096;   // candidates kept per part

// Sampled cutoff of a row: 32 blocks of 64 scores spread over the row give
// a conservative lower bound lo for tau (the sample's rank-r 13-bit bin, r
// chosen so that about 2m keys are expected at or above it).  hist (kBins1,
// zero on entry) is zero again on return.  A row of fewer than 64 scores has
// no room for the sample blocks: its cutoff is 0, the lowest key, so every
// score becomes a candidate (n < 64 fits any candidate list).  n is
// block-uniform, so the early return keeps the barriers uniform.
// Sample indices: block blk starts at floor(blk (n - 64) / 31) in [0, n - 64]
// and its 64 scores end at most at n - 1.
__device__ __forceinline__ uint32_t sampled_cutoff(const RowSplit& row, int n, int m, uint32_t* hist, Shared& sh) {
  if (n < 64) return 0u;
  const int t = threadIdx.x;
  const int blk = t >> 5;
  const int e0 = (int)(((int64_t)blk * (n - 64)) / 31) + 2 * (t & 31);
  atomicAdd(&hist[order_key(row.x[e0]) >> kShift1], 1u);
  atomicAdd(&hist[order_key(row.x[e0 + 1]) >> kShift1], 1u);
  __syncthreads();
  const uint32_t r = (uint32_t)min(2048ll, ((int64_t)2 * m * 2048 + n - 1) / n);
  find_bin(hist, kBins1, r, sh);
  const uint32_t lo = sh.bin << kShift1;
  for (int j = t; j < kBins1; j += kThreads) hist[j] = 0;
  return lo;
}

// Appends every key >= lo of the row's vector elements [q0, q1) (float4
// units), plus the scalar head (head) and tail (tail) elements, with its
// index, to the LDS candidate list (sh.ncand counts all of them, also past
// cap).  One wave-level append per iteration: each lane marks its
// candidates among its 4 x 4 scores, the wave forms the prefix of the
// counts from ballots, and one LDS atomic reserves the wave's slots.
__device__ __forceinline__ void collect_range(const RowSplit& row, int q0, int q1, bool head, bool tail_part,
                                              uint32_t lo, uint32_t* ckey, uint32_t* cidx, int cap, Shared& sh) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int iters = (q1 - q0 + kThreads * kUnroll - 1) / (kThreads * kUnroll);
  for (int it = 0; it < iters; ++it) {
    float4 v[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int q = q0 + (it * kUnroll + u) * kThreads + t;
      ok[u] = q < q1;
      v[u] = row.xv[ok[u] ? q : 0];
    }
    uint32_t keys[4 * kUnroll];
    uint32_t cm = 0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      keys[4 * u + 0] = order_key(v[u].x);
      keys[4 * u + 1] = order_key(v[u].y);
      keys[4 * u + 2] = order_key(v[u].z);
      keys[4 * u + 3] = order_key(v[u].w);
#pragma unroll
      for (int c = 0; c < 4; ++c) cm |= (ok[u] && keys[4 * u + c] >= lo ? 1u : 0u) << (4 * u + c);
    }
    uint32_t total;
    const uint32_t pre = wave_prefix_small((uint32_t)__popc(cm), total);
    if (total != 0) {   // wave-uniform
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&sh.ncand, total);
      base = __shfl(base, 0, 64);
      uint32_t pos = base + pre;
#pragma unroll
      for (int j = 0; j < 4 * kUnroll; ++j) {
        if ((cm >> j) & 1u) {
          if (pos < (uint32_t)cap) {
            ckey[pos] = keys[j];
            cidx[pos] = (uint32_t)(row.h + 4 * (q0 + (it * kUnroll + (j >> 2)) * kThreads + t) + (j & 3));
          }
          ++pos;
        }
      }
    }
  }
  auto one = [&](int e) {
    const uint32_t key = order_key(row.x[e]);
    if (key >= lo) {
      const uint32_t pos = atomicAdd(&sh.ncand, 1u);
      if (pos < (uint32_t)cap) { ckey[pos] = key; cidx[pos] = (uint32_t)e; }
    }
  };
  if (head && t < row.h) one(t);
  if (tail_part && t >= 4 && t - 4 < row.n - row.tail0) one(row.tail0 + t - 4);
}

// Collection half of the split top-k: part f of a row (nparts per row, row
// b * rows + i = blockIdx.x / nparts) takes the row's sampled cutoff (every
// part computes the same one) and collects the keys at or above it among
// its share of the row into the workspace.  Short rows (n <= k) write a
// zero count; the merge kernel handles them.
__global__ void __launch_bounds__(kThreads) topk_collect_kernel(TopkArgs a, Parts parts) {
  extern __shared__ uint32_t lds[];
  __shared__ Shared sh;
  const int t = threadIdx.x;
  const int f = blockIdx.x % parts.nparts;
  const int rowid = blockIdx.x / parts.nparts;
  const int b = rowid / a.rows, i = rowid % a.rows;
  const int n = min(row_pos_base(a.pk, b, a.S, a.pos0) + i + 1, a.S);
  const int m = min(a.k, n);
  uint32_t* cnt = parts.cnt + (int64_t)rowid * parts.nparts + f;
  if (n <= a.k) {
    if (t == 0) *cnt = 0u;
    return;
  }
  const RowSplit row(a.scores + ((int64_t)b * a.sc_rows_b + i) * a.ld, n);
  uint32_t* hist = lds;
  uint32_t* ckey = hist + kBins1;
  uint32_t* cidx = ckey + kCapPart;
  for (int j = t; j < kBins1; j += kThreads) hist[j] = 0;
  if (t == 0) sh.ncand = 0;
  __syncthreads();
  const uint32_t lo = sampled_cutoff(row, n, m, hist, sh);
  const int q0 = (int)((int64_t)row.nq * f / parts.nparts), q1 = (int)((int64_t)row.nq * (f + 1) / parts.nparts);
  collect_range(row, q0, q1, f == 0, f == parts.nparts - 1, lo, ckey, cidx, kCapPart, sh);
  __syncthreads();
  const uint32_t nc = sh.ncand;
  const int64_t base = ((int64_t)rowid * parts.nparts + f) * kCapPart;
  for (int j = t; j < (int)min(nc, (uint32_t)kCapPart); j += kThreads) {
    parts.key[base + j] = ckey[j];
    parts.idx[base + j] = cidx[j];
  }
  if (t == 0) *cnt = nc;
}

// The selection of one row (blockIdx.x = b * rows + i).  kParts: the
// candidates come from topk_collect_kernel's parts when they are usable
// (no part overflowed and m <= total <= cap), else the row takes the
// two-pass fallback; otherwise the row is sampled and collected here.
template <bool kParts>
__device__ __forceinline__ void topk_row(const TopkArgs& a, int cap, const Parts& parts) {
  extern __shared__ uint32_t lds[];
  __shared__ Shared sh;
  const int t = threadIdx.x;
  const int b = blockIdx.x / a.rows;
  const int i = blockIdx.x % a.rows;
  const int n = min(row_pos_base(a.pk, b, a.S, a.pos0) + i + 1, a.S);
  const int m = min(a.k, n);
  int32_t* out = a.idx + ((int64_t)b * a.idx_rows_b + i) * a.k;
  if (n <= a.k) {   // short row: every candidate is selected
    for (int j = t; j < a.k; j += kThreads) out[j] = j < n ? j : -1;
    return;
  }
  const RowSplit row(a.scores + ((int64_t)b * a.sc_rows_b + i) * a.ld, n);
  const int nwords = (n + 31) >> 5;
  const int words_max = (a.S + 31) >> 5;
  uint32_t* hist = lds;                  // kBins1 (reused for digits 2, 3)
  uint32_t* selbm = hist + kBins1;       // nwords
  uint32_t* tiebm = selbm + words_max;   // nwords
  uint32_t* ckey = tiebm + words_max;    // cap
  uint32_t* cidx = ckey + cap;           // cap

  for (int j = t; j < kBins1; j += kThreads) hist[j] = 0;
  for (int j = t; j < nwords; j += kThreads) { selbm[j] = 0; tiebm[j] = 0; }
  if (t == 0) sh.ncand = 0;
  __syncthreads();

  // Digits 2 and 3 of tau among the candidate list (every key of bin b1 is
  // on it; keys of other bins are filtered out), then the marks: keys above
  // tau into the bitmap, keys equal to tau into the tie bitmap.
  uint32_t tau, need;
  auto select_candidates = [&](int nc, uint32_t b1, uint32_t rank1) {
    for (int j = t; j < kBins2; j += kThreads) hist[j] = 0;
    __syncthreads();
    for (int c = t; c < nc; c += kThreads)
      if ((ckey[c] >> kShift1) == b1) atomicAdd(&hist[(ckey[c] >> kShift2) & (kBins2 - 1)], 1u);
    __syncthreads();
    find_bin(hist, kBins2, rank1, sh);
    const uint32_t pre = (b1 << (kShift1 - kShift2)) | sh.bin;
    const uint32_t rank2 = rank1 - sh.above;
    for (int j = t; j < kBins3; j += kThreads) hist[j] = 0;
    __syncthreads();
    for (int c = t; c < nc; c += kThreads)
      if ((ckey[c] >> kShift2) == pre) atomicAdd(&hist[ckey[c] & (kBins3 - 1)], 1u);
    __syncthreads();
    find_bin(hist, kBins3, rank2, sh);
    tau = (pre << kShift2) | sh.bin;
    need = rank2 - sh.above;
    for (int c = t; c < nc; c += kThreads) {
      const uint32_t key = ckey[c];
      if (key > tau) set_bit(selbm, (int)cidx[c]);
      else if (key == tau) set_bit(tiebm, (int)cidx[c]);
    }
  };

  // ---- one pass with a sampled cutoff (or the parts' candidates): if
  // between m and cap keys were collected, tau is the m-th largest candidate
  // and the selection is exact; otherwise the two-pass radix select below
  // runs.
  bool done = false;
  {
    if constexpr (kParts) {
      const int64_t pr = (int64_t)blockIdx.x * parts.nparts;
      uint32_t tot = 0;
      bool over = false;
      for (int f = 0; f < parts.nparts; ++f) {
        const uint32_t c = parts.cnt[pr + f];
        tot += c;
        over = over || c > (uint32_t)kCapPart;
      }
      const bool use = !over && tot >= (uint32_t)m && tot <= (uint32_t)cap;   // block-uniform
      if (use) {
        uint32_t off = 0;
        for (int f = 0; f < parts.nparts; ++f) {
          const uint32_t c = parts.cnt[pr + f];
          const int64_t base = (pr + f) * kCapPart;
          for (int j = t; j < (int)c; j += kThreads) {
            ckey[off + j] = parts.key[base + j];
            cidx[off + j] = parts.idx[base + j];
          }
          off += c;
        }
      }
      if (t == 0) sh.ncand = use ? tot : (uint32_t)cap + 1u;
    } else {
      const uint32_t lo = sampled_cutoff(row, n, m, hist, sh);
      collect_range(row, 0, row.nq, true, true, lo, ckey, cidx, cap, sh);
    }
    __syncthreads();
    const uint32_t nc = sh.ncand;
    if (nc >= (uint32_t)m && nc <= (uint32_t)cap) {   // block-uniform
      for (int c = t; c < (int)nc; c += kThreads) atomicAdd(&hist[ckey[c] >> kShift1], 1u);
      __syncthreads();
      find_bin(hist, kBins1, (uint32_t)m, sh);
      const uint32_t b1 = sh.bin;
      const uint32_t rank1 = (uint32_t)m - sh.above;
      select_candidates((int)nc, b1, rank1);
      done = true;
    } else {
      if (t == 0) sh.ncand = 0;
      __syncthreads();
    }
  }

  if (!done) {
    // ---- pass 1: digit-1 histogram
    scan_row(
        row, [&](int, uint32_t key, bool ok) { if (ok) atomicAdd(&hist[key >> kShift1], 1u); },
        [&](int, uint32_t key) { atomicAdd(&hist[key >> kShift1], 1u); });
    __syncthreads();
    find_bin(hist, kBins1, (uint32_t)m, sh);
    const uint32_t b1 = sh.bin;
    const uint32_t rank1 = (uint32_t)m - sh.above;   // rank of tau inside bin b1
    const uint32_t c1 = hist[b1];
    __syncthreads();
    if (c1 <= (uint32_t)cap) {
      // ---- pass 2: mark keys above bin b1, collect bin b1
      scan_row(
          row,
          [&](int e, uint32_t key, bool ok) {
            const uint32_t d = key >> kShift1;
            if (ok && d > b1) set_bit(selbm, e);
            append_wave(ok && d == b1, key, (uint32_t)e, ckey, cidx, cap, sh);
          },
          [&](int e, uint32_t key) {
            const uint32_t d = key >> kShift1;
            if (d > b1) set_bit(selbm, e);
            else if (d == b1) {
              const uint32_t pos = atomicAdd(&sh.ncand, 1u);
              if (pos < (uint32_t)cap) { ckey[pos] = key; cidx[pos] = (uint32_t)e; }
            }
          });
      __syncthreads();
      select_candidates((int)min(sh.ncand, (uint32_t)cap), b1, rank1);   // == c1 candidates
    } else {
      // ---- wide bin: resolve digits 2 and 3 with extra passes over the row
      for (int j = t; j < kBins2; j += kThreads) hist[j] = 0;
      __syncthreads();
      auto h2 = [&](int, uint32_t key) {
        if ((key >> kShift1) == b1) atomicAdd(&hist[(key >> kShift2) & (kBins2 - 1)], 1u);
      };
      scan_row(row, [&](int e, uint32_t key, bool ok) { if (ok) h2(e, key); }, h2);
      __syncthreads();
      find_bin(hist, kBins2, rank1, sh);
      const uint32_t pre = (b1 << (kShift1 - kShift2)) | sh.bin;
      const uint32_t rank2 = rank1 - sh.above;
      __syncthreads();
      for (int j = t; j < kBins3; j += kThreads) hist[j] = 0;
      __syncthreads();
      auto h3 = [&](int, uint32_t key) {
        if ((key >> kShift2) == pre) atomicAdd(&hist[key & (kBins3 - 1)], 1u);
      };
      scan_row(row, [&](int e, uint32_t key, bool ok) { if (ok) h3(e, key); }, h3);
      __syncthreads();
      find_bin(hist, kBins3, rank2, sh);
      tau = (pre << kShift2) | sh.bin;
      need = rank2 - sh.above;
      auto mark = [&](int e, uint32_t key) {
        if (key > tau) set_bit(selbm, e);
        else if (key == tau) set_bit(tiebm, e);
      };
      scan_row(row, [&](int e, uint32_t key, bool ok) { if (ok) mark(e, key); }, mark);
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

__global__ void __launch_bounds__(kThreads) topk_kernel(TopkArgs a, int cap) { topk_row<false>(a, cap, Parts{}); }

__global__ void __launch_bounds__(kThreads) topk_merge_kernel(TopkArgs a, int cap, Parts parts) {
  topk_row<true>(a, cap, parts);
}

// Candidate capacity of the single-row selection: what the LDS budget
// leaves, at most kMaxCand (at the largest supported S this is still ~7900,
// above any plausible cutoff bin).
int row_cap(const TopkArgs& a, size_t& lds) {
  const size_t words = (size_t)((a.S + 31) >> 5);
  const size_t fixed = (kBins1 + 2 * words) * sizeof(uint32_t);
  const int cap = (int)min((size_t)kMaxCand, (kDynLds - fixed) / (2 * sizeof(uint32_t)));
  lds = fixed + 2 * (size_t)cap * sizeof(uint32_t);
  return cap;
}

hipError_t set_dyn_lds(const void* fn) {
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kDynLds);
}

}  // namespace

int topk_max_kv() { return kMaxKV; }

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.rows <= 0 || a.B <= 0) return hipSuccess;
  size_t lds = 0;
  const int cap = row_cap(a, lds);
  static DeviceOnce attr;
  const hipError_t ae = (hipError_t)device_once(attr, (int)hipErrorInvalidDevice,
                                                [](int) { return (int)set_dyn_lds((const void*)topk_kernel); });
  if (ae != hipSuccess) return ae;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)(a.B * a.rows)), dim3(kThreads), lds, st, a, cap);
  return hipGetLastError();
}

int topk_split_parts(int64_t rows_total, int S) {
  // Few long rows leave most CUs idle with one workgroup per row: spread
  // each row's collection over up to 8 workgroups (about 256 in all).
  if (S < 16384 || rows_total <= 0 || rows_total > 128) return 1;
  const int64_t p = 256 / rows_total;
  return (int)(p < 2 ? 2 : p > 8 ? 8 : p);
}

size_t topk_split_bytes(int64_t rows_total, int nparts) {
  if (nparts <= 1) return 0;
  const size_t n = (size_t)rows_total * nparts;
  return (n * sizeof(uint32_t) + 255) / 256 * 256 + 2 * n * kCapPart * sizeof(uint32_t);
}

hipError_t launch_topk_split(const TopkArgs& a, int nparts, void* ws, hipStream_t st) {
  if (a.rows <= 0 || a.B <= 0) return hipSuccess;
  if (nparts <= 1) return launch_topk(a, st);
  const size_t n = (size_t)a.B * a.rows * nparts;
  Parts parts;
  parts.cnt = (uint32_t*)ws;
  parts.key = (uint32_t*)((char*)ws + (n * sizeof(uint32_t) + 255) / 256 * 256);
  parts.idx = parts.key + n * kCapPart;
  parts.nparts = nparts;
  size_t lds = 0;
  const int cap = row_cap(a, lds);
  static DeviceOnce attr;
  const hipError_t ae = (hipError_t)device_once(attr, (int)hipErrorInvalidDevice, [](int) {
    hipError_t e = set_dyn_lds((const void*)topk_collect_kernel);
    if (e == hipSuccess) e = set_dyn_lds((const void*)topk_merge_kernel);
    return (int)e;
  });
  if (ae != hipSuccess) return ae;
  const size_t lds_collect = (kBins1 + 2 * (size_t)kCapPart) * sizeof(uint32_t);
  hipLaunchKernelGGL(topk_collect_kernel, dim3((unsigned)n), dim3(kThreads), lds_collect, st, a, parts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)(a.B * a.rows)), dim3(kThreads), lds, st, a, cap, parts);
  return hipGetLastError();
}

}  // namespace dsa
