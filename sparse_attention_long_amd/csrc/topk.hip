// Per-row top-k selection (page "DeepSeek-V3.2: sparse attention, scaled RL
// and synthetic agent environments": the selected set S_t of Sec. 1.1 /
// Eq. (4); rows shorter than k keep everything, Sec. 5.1; equal scores at
// the cutoff are legitimate, Sec. 5.2 near Eq. (18) -- here they go to the
// lower index).
//
// One workgroup of 512 threads per row.  Scores are mapped to
// order-preserving 32-bit keys (NaN lowest, -0 == +0).  The selection is
// fixed by tau, the m-th largest key, and `need`, the number of keys equal
// to tau that are kept (the lowest-indexed ones):
//   Sampled single pass (the usual path): 2048 scores (32 blocks of 64
//          spread over the row) give a provisional cutoff lo, the lower
//          edge of the 13-bit bin (sign, exponent, 4 mantissa bits) that
//          holds the sample's rank-r key, with r set so that about 2m keys
//          of the row are expected at or above lo.  One pass over the row
//          collects every key >= lo, with its index, into an LDS candidate
//          list in ascending index order: in each iteration a thread takes
//          16 consecutive scores, and one block-wide prefix sum of the
//          threads' counts places their candidates.  If between m and kCap
//          keys were collected, tau and need come from a radix select over
//          the candidates.
//   Fallback (the sample missed): pass 1 builds the histogram of the 13-bit
//          digit over the whole row and fixes tau's bin b1.  If the keys at
//          or above b1 fit the list, pass 2 collects them (in order) and
//          the selection proceeds as above; a wider bin takes one more pass
//          per remaining digit to fix tau and need, and a last ordered pass
//          writes the selection.
// Because the candidates are in index order, the selection is written by an
// order-keeping compaction (every key above tau, then the first `need` keys
// equal to tau, in index order) with no bitmap and no sort.  The 13-bit
// histogram and the candidate list share their LDS, so a row needs about
// 70 KB and two rows run on a CU at once (512 threads each, at most 128
// VGPRs): one row's serial phases overlap the other's streaming.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxKV = 262144;
constexpr int kShift1 = 19;                 // digit 1 = key bits 31..19
constexpr int kBins1 = 1 << (32 - kShift1); // 8192
constexpr int kShift2 = 9;                  // digit 2 = key bits 18..9
constexpr int kBins2 = 1 << (kShift1 - kShift2);   // 1024
constexpr int kBins3 = 1 << kShift2;        // digit 3 = key bits 8..0: 512
constexpr int kCap = 8192;                  // candidates of a row in LDS
constexpr int kSlice = kCap / kThreads;     // candidates per thread in the selection
constexpr int kVec = 4;                     // float4s per thread and iteration: 16 consecutive scores
constexpr int kCapPart = 4096;              // candidates per part of the split top-k

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (x != x) return 0u;                    // NaN below everything
  if (u == 0x80000000u) u = 0u;             // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct Shared {
  uint32_t scan[2][kWaves];   // block_scan's wave totals, two buffers
  uint32_t bin, above, total, flag;
};

// LDS of a row's workgroup.  The 13-bit histogram (cutoff search, fallback
// pass 1) and the candidate list are never needed at the same time.
template <int CAP>
struct RowLds {
  union {
    uint32_t hist1[kBins1];
    struct {
      uint32_t key[CAP];
      uint32_t idx[CAP];
    } c;
  } u;
  uint32_t hist2[kBins2];   // digits 2 and 3, the 8-bit digits, reductions
  Shared sh;
};
static_assert(2 * kCap >= kBins1 && 2 * kCapPart >= kBins1, "the histogram fits the candidate space");
static_assert(2048 % kThreads == 0 && kThreads >= 256 && kCap % kThreads == 0, "sample and slice shapes");
static_assert(kCap < 65536, "emission packs two candidate counts in one word");

__device__ __forceinline__ void zero(uint32_t* p, int n) {
  for (int j = threadIdx.x; j < n; j += kThreads) p[j] = 0u;
}

// Exclusive prefix sum over the block in thread order, and the block total.
// One barrier: the wave totals go to buffer `buf`, and a scan that follows
// another with no barrier in between must use the other buffer (a wave can
// then only overwrite a buffer after every wave has passed the barrier of
// the scan in between, i.e. has finished reading it).
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t& total, Shared& sh, int buf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) sh.scan[buf][wave] = x;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t s = sh.scan[buf][w];
    pre += w < wave ? s : 0u;
    tot += s;
  }
  total = tot;
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
  uint32_t tot;
  const uint32_t excl = block_scan(local, tot, sh, 0);   // a barrier follows
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

// Calls f(key, valid) for every element of the row, in no particular order
// (histogram passes): 16-byte loads, consecutive lanes on consecutive
// float4s, four per thread in flight.  The vector part runs the same number
// of iterations in every thread (block-uniform), so f may use wave-wide
// operations.  The < 8 head and tail elements are visited by threads 0..7
// afterwards with a per-thread call g(key).
template <class F, class G>
__device__ __forceinline__ void scan_row(const RowSplit& r, F&& f, G&& g) {
  const int t = threadIdx.x;
  const int iters = (r.nq + kThreads * kVec - 1) / (kThreads * kVec);
  for (int it = 0; it < iters; ++it) {
    float4 v[kVec];
    bool ok[kVec];
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      const int q = (it * kVec + u) * kThreads + t;
      ok[u] = q < r.nq;
      v[u] = r.xv[ok[u] ? q : 0];
    }
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      f(order_key(v[u].x), ok[u]);
      f(order_key(v[u].y), ok[u]);
      f(order_key(v[u].z), ok[u]);
      f(order_key(v[u].w), ok[u]);
    }
  }
  if (t < r.h) g(order_key(r.x[t]));
  if (t >= 4 && t - 4 < r.n - r.tail0) g(order_key(r.x[r.tail0 + t - 4]));
}

// The ordered passes: iteration it of a range of float4s starting at q0
// gives thread t the float4s q0 + (it * kThreads + t) * kVec + u, u < kVec:
// 16 consecutive scores, so that thread order is element order.
// ordered_loads issues the loads; keys_of maps them to keys (valid: inside
// [q0, q1)); ordered_keys does both.
__device__ __forceinline__ void ordered_loads(const RowSplit& r, int q0, int q1, int it, float4 (&v)[kVec]) {
  const int qb = q0 + (it * kThreads + (int)threadIdx.x) * kVec;
#pragma unroll
  for (int u = 0; u < kVec; ++u) v[u] = r.xv[qb + u < q1 ? qb + u : q0];
}

__device__ __forceinline__ int keys_of(const RowSplit& r, int q0, int q1, int it, const float4 (&v)[kVec],
                                       uint32_t (&keys)[4 * kVec], uint32_t& valid) {
  const int qb = q0 + (it * kThreads + (int)threadIdx.x) * kVec;
  valid = 0;
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    keys[4 * u + 0] = order_key(v[u].x);
    keys[4 * u + 1] = order_key(v[u].y);
    keys[4 * u + 2] = order_key(v[u].z);
    keys[4 * u + 3] = order_key(v[u].w);
    valid |= (qb + u < q1 ? 0xFu : 0u) << (4 * u);
  }
  return r.h + 4 * qb;   // element index of keys[0]
}

__device__ __forceinline__ int ordered_keys(const RowSplit& r, int q0, int q1, int it, uint32_t (&keys)[4 * kVec],
                                            uint32_t& valid) {
  float4 v[kVec];
  ordered_loads(r, q0, q1, it, v);
  return keys_of(r, q0, q1, it, v, keys, valid);
}

// Collects the keys >= lo of float4s [q0, q1) (and, for head / tail, of the
// row's scalar head and tail) into ckey / cidx in element order; returns
// their count (entries past cap are counted, not stored).  Each iteration's
// loads are issued before the previous iteration's block scan, so the scan's
// barriers overlap the memory latency.
__device__ uint32_t collect_ordered(const RowSplit& r, int q0, int q1, bool head, bool tail, uint32_t lo,
                                    uint32_t* ckey, uint32_t* cidx, uint32_t cap, Shared& sh) {
  const int t = threadIdx.x;
  uint32_t base = 0;
  if (head && r.h > 0) {
    if (t == 0) {
      uint32_t c = 0;
      for (int e = 0; e < r.h; ++e) {
        const uint32_t key = order_key(r.x[e]);
        if (key >= lo) {
          if (c < cap) { ckey[c] = key; cidx[c] = (uint32_t)e; }
          ++c;
        }
      }
      sh.total = c;
    }
    __syncthreads();
    base = sh.total;
    __syncthreads();
  }
  const int iters = (q1 - q0 + kThreads * kVec - 1) / (kThreads * kVec);
  float4 nv[kVec];
  if (iters > 0) ordered_loads(r, q0, q1, 0, nv);
  for (int it = 0; it < iters; ++it) {
    float4 v[kVec];
#pragma unroll
    for (int u = 0; u < kVec; ++u) v[u] = nv[u];
    if (it + 1 < iters) ordered_loads(r, q0, q1, it + 1, nv);
    uint32_t keys[4 * kVec], valid;
    const int e0 = keys_of(r, q0, q1, it, v, keys, valid);
    uint32_t cm = 0;
#pragma unroll
    for (int j = 0; j < 4 * kVec; ++j) cm |= (keys[j] >= lo ? 1u : 0u) << j;
    cm &= valid;
    uint32_t tot;
    uint32_t pos = base + block_scan((uint32_t)__popc(cm), tot, sh, it & 1);
#pragma unroll
    for (int j = 0; j < 4 * kVec; ++j)
      if ((cm >> j) & 1u) {
        if (pos < cap) { ckey[pos] = keys[j]; cidx[pos] = (uint32_t)(e0 + j); }
        ++pos;
      }
    base += tot;
  }
  if (tail && r.tail0 < r.n) {
    if (t == 0) {
      uint32_t c = base;
      for (int e = r.tail0; e < r.n; ++e) {
        const uint32_t key = order_key(r.x[e]);
        if (key >= lo) {
          if (c < cap) { ckey[c] = key; cidx[c] = (uint32_t)e; }
          ++c;
        }
      }
      sh.total = c;
    }
    __syncthreads();
    base = sh.total;
    __syncthreads();
  }
  return base;
}

// A thread's slice of the candidate list, in registers: entries
// [t * per, t * per + n) with per = ceil(nc / kThreads) <= kSlice.
struct Slice {
  uint32_t key[kSlice], idx[kSlice];
  uint32_t n;
};

__device__ __forceinline__ void load_slice(const uint32_t* ckey, const uint32_t* cidx, uint32_t nc, Slice& s) {
  const uint32_t per = (nc + kThreads - 1) / kThreads;
  const uint32_t j0 = min((uint32_t)threadIdx.x * per, nc);
  s.n = min(j0 + per, nc) - j0;
#pragma unroll
  for (int u = 0; u < kSlice; ++u) {
    const bool ok = (uint32_t)u < s.n;
    s.key[u] = ok ? ckey[j0 + u] : 0u;
    s.idx[u] = ok ? cidx[j0 + u] : 0u;
  }
}

// tau, the m-th largest key of the candidates held in the threads' slices
// (m <= their number), and need, how many keys equal to tau are selected.
// The bits every candidate shares (above the highest bit where the largest
// and smallest keys differ) are fixed at once; the rest are resolved 8 at
// a time from the top, with a 256-bin histogram in `hist`.
__device__ void select_tau(const Slice& s, uint32_t m, uint32_t* hist, uint32_t* wide, Shared& sh, uint32_t& tau,
                           uint32_t& need) {
  const int t = threadIdx.x;
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int u = 0; u < kSlice; ++u)
    if ((uint32_t)u < s.n) {
      kmax = max(kmax, s.key[u]);
      kmin = min(kmin, s.key[u]);
    }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, d, kWave));
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, d, kWave));
  }
  if ((t & 63) == 0) {
    hist[t >> 6] = kmax;
    hist[kWaves + (t >> 6)] = kmin;
  }
  __syncthreads();
  kmax = 0u;
  kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    kmax = max(kmax, hist[w]);
    kmin = min(kmin, hist[kWaves + w]);
  }
  __syncthreads();
  int hi = kmax == kmin ? -1 : 31 - __clz(kmax ^ kmin);   // highest differing bit
  uint32_t pmask = hi < 0 ? 0xFFFFFFFFu : hi >= 31 ? 0u : ~((2u << hi) - 1u);
  uint32_t prefix = kmax & pmask, rank = m;
  // First round, when more than 8 bits vary: an 11-bit digit over up to 2048
  // bins in `wide` (the candidate list's space, free once the slices are
  // loaded).  The top digit below the common prefix is the crowded one
  // (most candidates lie just above the cutoff); 8 times as many bins keep
  // their LDS atomics from piling onto a few addresses, and the round
  // covers 3 more bits.
  if (hi >= 8) {
    const int lo_bit = hi - 10 > 0 ? hi - 10 : 0;
    const int nbins = 2 << (hi - lo_bit);
    const uint32_t dmask = (uint32_t)nbins - 1u;
    zero(wide, nbins);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kSlice; ++u)
      if ((uint32_t)u < s.n) atomicAdd(&wide[(s.key[u] >> lo_bit) & dmask], 1u);
    __syncthreads();
    find_bin(wide, nbins, rank, sh);   // ends with a barrier
    prefix |= sh.bin << lo_bit;
    pmask |= dmask << lo_bit;
    rank -= sh.above;
    hi = lo_bit - 1;
  }
  // Two 256-bin histograms alternate between the remaining rounds: a round
  // fills one and clears the other, and wave 0 alone finds the bin, so a
  // round needs two barriers.
  uint32_t* hc = hist;
  uint32_t* hn = hist + 256;
  if (t < 256) hc[t] = 0u;
  __syncthreads();
  while (hi >= 0) {   // block-uniform
    const int lo_bit = max(hi - 7, 0);
    const uint32_t dmask = (2u << (hi - lo_bit)) - 1u;
#pragma unroll
    for (int u = 0; u < kSlice; ++u)
      if ((uint32_t)u < s.n && (s.key[u] & pmask) == prefix) atomicAdd(&hc[(s.key[u] >> lo_bit) & dmask], 1u);
    if (t < 256) hn[t] = 0u;
    __syncthreads();
    if (t < kWave) {
      // lane l owns bins 255 - 4l - j (j < 4): lane order is bin order from the top
      uint32_t c[4], local = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hc[255 - 4 * t - j];
        local += c[j];
      }
      uint32_t incl = local;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t y = __shfl_up(incl, d, kWave);
        if (t >= d) incl += y;
      }
      uint32_t cum = incl - local;
      if (local > 0 && cum < rank && rank <= incl) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (cum + c[j] >= rank) {
            sh.bin = (uint32_t)(255 - 4 * t - j);
            sh.above = cum;
            break;
          }
          cum += c[j];
        }
      }
    }
    __syncthreads();
    prefix |= sh.bin << lo_bit;
    pmask |= dmask << lo_bit;
    rank -= sh.above;
    hi = lo_bit - 1;
    uint32_t* tmp = hc;
    hc = hn;
    hn = tmp;
  }
  tau = prefix;
  need = rank;
}

// Writes the selection from the slices (which are in element order): every
// key above tau and the first `need` keys equal to tau, in element order.
// One block scan gives each thread both the keys above tau and the keys
// equal to tau held by the threads before it (each count is below 2^16,
// packed in one word); a kept key's slot is then (keys above tau before it)
// + min(keys equal to tau before it, need).
__device__ void emit_slices(const Slice& s, uint32_t tau, uint32_t need, uint32_t m, int32_t* out, Shared& sh) {
  uint32_t above = 0, ties = 0;
#pragma unroll
  for (int u = 0; u < kSlice; ++u) {
    const bool in = (uint32_t)u < s.n;
    above += in && s.key[u] > tau ? 1u : 0u;
    ties += in && s.key[u] == tau ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t before = block_scan(above | (ties << 16), tot, sh, 0);
  uint32_t a = before & 0xFFFFu, t = before >> 16;
#pragma unroll
  for (int u = 0; u < kSlice; ++u) {
    if ((uint32_t)u >= s.n) continue;
    if (s.key[u] > tau) {
      const uint32_t pos = a + min(t, need);
      if (pos < m) out[pos] = (int32_t)s.idx[u];
      ++a;
    } else if (s.key[u] == tau) {
      if (t < need && a + t < m) out[a + t] = (int32_t)s.idx[u];
      ++t;
    }
  }
}

// The last pass of the wide-bin fallback: writes, in element order, every
// element whose key is above tau and the first `need` with key tau.
__device__ void write_selection(const RowSplit& r, uint32_t tau, uint32_t need, uint32_t m, int32_t* out,
                                Shared& sh) {
  const int t = threadIdx.x;
  uint32_t base = 0, tbase = 0;   // selected and ties so far (block-uniform)
  auto serial = [&](int e0, int e1) {   // thread 0 only
    for (int e = e0; e < e1; ++e) {
      const uint32_t key = order_key(r.x[e]);
      if (key > tau || (key == tau && tbase++ < need)) {
        if (base < m) out[base] = e;
        ++base;
      }
    }
  };
  if (r.h > 0) {
    if (t == 0) {
      serial(0, r.h);
      sh.bin = base;
      sh.above = tbase;
    }
    __syncthreads();
    base = sh.bin;
    tbase = sh.above;
    __syncthreads();
  }
  const int iters = (r.nq + kThreads * kVec - 1) / (kThreads * kVec);
  for (int it = 0; it < iters; ++it) {
    uint32_t keys[4 * kVec], valid;
    const int e0 = ordered_keys(r, 0, r.nq, it, keys, valid);
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < 4 * kVec; ++j) {
      gt |= (keys[j] > tau ? 1u : 0u) << j;
      eq |= (keys[j] == tau ? 1u : 0u) << j;
    }
    gt &= valid;
    eq &= valid;
    uint32_t ttot;
    const uint32_t tpre = tbase + block_scan((uint32_t)__popc(eq), ttot, sh, 0);
    // this thread's kept ties: those whose rank tpre + (ties before) < need
    uint32_t keepm = gt, tr = tpre;
#pragma unroll
    for (int j = 0; j < 4 * kVec; ++j)
      if ((eq >> j) & 1u) keepm |= (tr++ < need ? 1u : 0u) << j;
    uint32_t ktot;
    uint32_t pos = base + block_scan((uint32_t)__popc(keepm), ktot, sh, 1);
#pragma unroll
    for (int j = 0; j < 4 * kVec; ++j)
      if ((keepm >> j) & 1u) {
        if (pos < m) out[pos] = e0 + j;
        ++pos;
      }
    base += ktot;
    tbase += ttot;
  }
  if (r.tail0 < r.n && t == 0) serial(r.tail0, r.n);
  __syncthreads();
}

// Sampled cutoff of a row: 32 blocks of 64 scores spread over the row give
// a conservative lower bound lo for tau (the sample's rank-r 13-bit bin, r
// chosen so that about 2m keys are expected at or above it).  hist (kBins1)
// is cleared here, after the sample loads are issued, so that their latency
// overlaps the clearing.  A row of fewer than 64 scores has no room for the
// sample blocks: its cutoff is 0, the lowest key, so every score becomes a
// candidate (n < 64 fits any candidate list).  n is block-uniform, so the
// early return keeps the barriers uniform.
// Sample indices: block blk starts at floor(blk (n - 64) / 31) in [0, n - 64]
// and its 64 scores end at most at n - 1.
__device__ __forceinline__ uint32_t sampled_cutoff(const RowSplit& row, int n, int m, uint32_t* hist, Shared& sh) {
  if (n < 64) return 0u;
  constexpr int kPer = 2048 / kThreads;   // sample scores per thread
  constexpr int kTpb = 64 / kPer;         // threads per block of 64
  const int t = threadIdx.x;
  const int blk = t / kTpb;
  const int e0 = (int)(((int64_t)blk * (n - 64)) / 31) + kPer * (t % kTpb);
  float x[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) x[j] = row.x[e0 + j];
  zero(hist, kBins1);   // while the sample loads are in flight
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j) atomicAdd(&hist[order_key(x[j]) >> kShift1], 1u);
  __syncthreads();
  const uint32_t r = (uint32_t)min(2048ll, ((int64_t)2 * m * 2048 + n - 1) / n);
  find_bin(hist, kBins1, r, sh);
  return sh.bin << kShift1;
}

// Candidates of a row collected by the parts of topk_collect_kernel, each
// part's list in element order and the parts in row order.
struct Parts {
  uint32_t* cnt;   // [rows_total * nparts] keys each part found at or above its cutoff
  uint32_t* key;   // [rows_total * nparts * kCapPart]
  uint32_t* idx;
  int nparts;
};

// Collection half of the split top-k: part f of a row (nparts per row, row
// b * rows + i = blockIdx.x / nparts) takes the row's sampled cutoff (every
// part computes the same one) and collects the keys at or above it among
// its contiguous share of the row, in element order, into the workspace.
// Short rows (n <= k) write a zero count; the merge kernel handles them.
__global__ void __launch_bounds__(kThreads) topk_collect_kernel(TopkArgs a, Parts parts) {
  __shared__ RowLds<kCapPart> L;
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
  const uint32_t lo = sampled_cutoff(row, n, m, L.u.hist1, L.sh);
  const int q0 = (int)((int64_t)row.nq * f / parts.nparts), q1 = (int)((int64_t)row.nq * (f + 1) / parts.nparts);
  const uint32_t nc = collect_ordered(row, q0, q1, f == 0, f == parts.nparts - 1, lo, L.u.c.key, L.u.c.idx,
                                      kCapPart, L.sh);
  __syncthreads();
  const int64_t base = ((int64_t)rowid * parts.nparts + f) * kCapPart;
  for (int j = t; j < (int)min(nc, (uint32_t)kCapPart); j += kThreads) {
    parts.key[base + j] = L.u.c.key[j];
    parts.idx[base + j] = L.u.c.idx[j];
  }
  if (t == 0) *cnt = nc;
}

// The selection of one row (blockIdx.x = b * rows + i).  kParts: the
// candidates come from topk_collect_kernel's parts when they are usable (no
// part overflowed and m <= total <= kCap); otherwise, and without parts,
// the row is sampled and collected here, with the two-pass fallback.
template <bool kParts>
__device__ __forceinline__ void topk_row(const TopkArgs& a, const Parts& parts) {
  __shared__ RowLds<kCap> L;
  const int t = threadIdx.x;
  const int b = blockIdx.x / a.rows;
  const int i = blockIdx.x % a.rows;
  const int n = min(row_pos_base(a.pk, b, a.S, a.pos0) + i + 1, a.S);
  const uint32_t m = (uint32_t)min(a.k, n);
  int32_t* out = a.idx + ((int64_t)b * a.idx_rows_b + i) * a.k;
  if (n <= a.k) {   // short row: every candidate is selected
    for (int j = t; j < a.k; j += kThreads) out[j] = j < n ? j : -1;
    return;
  }
  const RowSplit row(a.scores + ((int64_t)b * a.sc_rows_b + i) * a.ld, n);
  uint32_t* ckey = L.u.c.key;
  uint32_t* cidx = L.u.c.idx;
  uint32_t nc = 0;
  bool have = false;   // block-uniform: [0, nc) of the list holds every key >= some cutoff, m <= nc <= kCap
  bool sliced = false;   // block-uniform: the slices already hold the list (loaded from the parts)
  Slice s;
  if constexpr (kParts) {
    // the parts' counts, one load per thread
    if (t < parts.nparts) L.hist2[t] = parts.cnt[(int64_t)blockIdx.x * parts.nparts + t];
    __syncthreads();
    if (t == 0) {
      uint32_t tot = 0;
      bool over = false;
      for (int f = 0; f < parts.nparts; ++f) {
        const uint32_t c = L.hist2[f];
        over = over || c > (uint32_t)kCapPart;
        L.hist2[kBins2 / 2 + f] = tot;   // the part's offset in the list
        tot += c;
      }
      L.sh.total = tot;
      L.sh.flag = !over && tot >= m && tot <= (uint32_t)kCap ? 1u : 0u;
    }
    __syncthreads();
    if (L.sh.flag) {
      // The list is the parts' lists back to back.  Each thread loads its
      // slice of it (the positions load_slice gives it) straight from the
      // parts, all loads in flight at once; part f's list starts at list
      // position off[f] and at workspace element (row * nparts + f) * kCapPart.
      nc = L.sh.total;
      const uint32_t* off = L.hist2 + kBins2 / 2;
      const int np = parts.nparts;
      const uint32_t per = (nc + kThreads - 1) / kThreads;
      const uint32_t j0 = min((uint32_t)t * per, nc);
      s.n = min(j0 + per, nc) - j0;
      const int64_t rowbase = (int64_t)blockIdx.x * np * kCapPart;
      int f = 0;
      uint32_t lo_f = 0u, hi_f = np > 1 ? off[1] : 0xFFFFFFFFu;   // part f spans list positions [lo_f, hi_f)
#pragma unroll
      for (int u = 0; u < kSlice; ++u) {
        const uint32_t j = j0 + u;
        const bool ok = (uint32_t)u < s.n;
        while (ok && j >= hi_f) {   // empty parts are skipped too
          ++f;
          lo_f = hi_f;
          hi_f = f + 1 < np ? off[f + 1] : 0xFFFFFFFFu;
        }
        const int64_t src = rowbase + (int64_t)f * kCapPart + (j - lo_f);
        s.key[u] = ok ? parts.key[src] : 0u;
        s.idx[u] = ok ? parts.idx[src] : 0u;
      }
      have = true;
      sliced = true;
    }
    __syncthreads();
  }
  if (!have) {
    const uint32_t lo = sampled_cutoff(row, n, (int)m, L.u.hist1, L.sh);
    nc = collect_ordered(row, 0, row.nq, true, true, lo, ckey, cidx, kCap, L.sh);
    have = nc >= m && nc <= (uint32_t)kCap;
  }
  if (!have) {
    // ---- pass 1: digit-1 histogram over the row (the list is discarded)
    __syncthreads();
    zero(L.u.hist1, kBins1);
    __syncthreads();
    uint32_t* h1 = L.u.hist1;
    scan_row(row, [&](uint32_t key, bool ok) { if (ok) atomicAdd(&h1[key >> kShift1], 1u); },
             [&](uint32_t key) { atomicAdd(&h1[key >> kShift1], 1u); });
    __syncthreads();
    find_bin(h1, kBins1, m, L.sh);
    const uint32_t b1 = L.sh.bin;
    const uint32_t above1 = L.sh.above;
    const uint32_t c1 = h1[b1];
    __syncthreads();
    if (above1 + c1 <= (uint32_t)kCap) {
      // ---- pass 2: collect every key at or above bin b1, in order
      nc = collect_ordered(row, 0, row.nq, true, true, b1 << kShift1, ckey, cidx, kCap, L.sh);
      have = true;   // nc == above1 + c1, which lies in [m, kCap]
    } else {
      // ---- wide bin: digits 2 and 3 with one pass each, then the selection
      uint32_t* h2 = L.hist2;
      zero(h2, kBins2);
      __syncthreads();
      scan_row(
          row, [&](uint32_t key, bool ok) { if (ok && (key >> kShift1) == b1) atomicAdd(&h2[(key >> kShift2) & (kBins2 - 1)], 1u); },
          [&](uint32_t key) { if ((key >> kShift1) == b1) atomicAdd(&h2[(key >> kShift2) & (kBins2 - 1)], 1u); });
      __syncthreads();
      const uint32_t rank1 = m - above1;
      find_bin(h2, kBins2, rank1, L.sh);
      const uint32_t pre = (b1 << (kShift1 - kShift2)) | L.sh.bin;
      const uint32_t rank2 = rank1 - L.sh.above;
      __syncthreads();
      zero(h2, kBins3);
      __syncthreads();
      scan_row(row, [&](uint32_t key, bool ok) { if (ok && (key >> kShift2) == pre) atomicAdd(&h2[key & (kBins3 - 1)], 1u); },
               [&](uint32_t key) { if ((key >> kShift2) == pre) atomicAdd(&h2[key & (kBins3 - 1)], 1u); });
      __syncthreads();
      find_bin(h2, kBins3, rank2, L.sh);
      const uint32_t tau = (pre << kShift2) | L.sh.bin;
      const uint32_t need = rank2 - L.sh.above;
      __syncthreads();
      write_selection(row, tau, need, m, out, L.sh);
    }
  }
  if (have) {
    if (!sliced) {
      __syncthreads();
      load_slice(ckey, cidx, nc, s);
    }
    __syncthreads();   // the list (or the part offsets) may now be overwritten: select_tau takes their space
    uint32_t tau, need;
    select_tau(s, m, L.hist2, L.u.hist1, L.sh, tau, need);
    emit_slices(s, tau, need, m, out, L.sh);
  }
  for (int j = (int)m + t; j < a.k; j += kThreads) out[j] = -1;
}

__global__ void __launch_bounds__(kThreads) topk_kernel(TopkArgs a) { topk_row<false>(a, Parts{}); }

__global__ void __launch_bounds__(kThreads) topk_merge_kernel(TopkArgs a, Parts parts) { topk_row<true>(a, parts); }

}  // namespace

int topk_max_kv() { return kMaxKV; }

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.rows <= 0 || a.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)(a.B * a.rows)), dim3(kThreads), 0, st, a);
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
  if (nparts > kBins2 / 2) return hipErrorInvalidValue;
  const size_t n = (size_t)a.B * a.rows * nparts;
  Parts parts;
  parts.cnt = (uint32_t*)ws;
  parts.key = (uint32_t*)((char*)ws + (n * sizeof(uint32_t) + 255) / 256 * 256);
  parts.idx = parts.key + n * kCapPart;
  parts.nparts = nparts;
  hipLaunchKernelGGL(topk_collect_kernel, dim3((unsigned)n), dim3(kThreads), 0, st, a, parts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)(a.B * a.rows)), dim3(kThreads), 0, st, a, parts);
  return hipGetLastError();
}

}  // namespace dsa
