// Locality counters of the selected sets (the analysis page "DeepSeek-V3.2:
// sparse attention, scaled RL and synthetic agent environments", Sec. 5.1:
// a row's selected cache entries may sit in a few contiguous pages or be
// spread over many, and a profiler should record the distinct pages, the
// contiguous runs and the hits per page of each row).
//
// Per row of a [B, T, k] selection (ascending token indices, entries < 0
// skipped): the number of distinct pages (token / page_size), the number of
// maximal runs of consecutive indices, and the largest number of selected
// tokens on one page.  One wave per row: the row and its page ids are staged
// in LDS, lane l summarises entries [l*per, (l+1)*per), and the 64 summaries
// are merged pairwise in 6 levels, always left block before right block (a
// run or a page segment may continue across a block border).
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kMaxK = 2048;

struct Block {
  int cnt;        // valid entries
  int first, last;
  int pfirst, plast;   // pages of first / last
  int runs, pages;
  int head, tail; // length of the first / last page segment
  int mx;         // longest page segment
};

__device__ __forceinline__ Block merge(const Block& x, const Block& y) {
  if (x.cnt == 0) return y;
  if (y.cnt == 0) return x;
  Block r;
  const bool run_join = y.first == x.last + 1;
  const bool page_join = y.pfirst == x.plast;
  r.cnt = x.cnt + y.cnt;
  r.first = x.first;
  r.last = y.last;
  r.pfirst = x.pfirst;
  r.plast = y.plast;
  r.runs = x.runs + y.runs - (run_join ? 1 : 0);
  r.pages = x.pages + y.pages - (page_join ? 1 : 0);
  const int joined = page_join ? x.tail + y.head : 0;
  r.head = (page_join && x.pages == 1) ? x.head + y.head : x.head;
  r.tail = (page_join && y.pages == 1) ? x.tail + y.tail : y.tail;
  r.mx = max(max(x.mx, y.mx), joined);
  return r;
}

__global__ void __launch_bounds__(kWave) gather_stats_kernel(const int32_t* idx, int32_t* stats, int64_t rows, int k,
                                                               int ps) {
  __shared__ int32_t row_s[kMaxK];
  __shared__ int32_t row_p[kMaxK];
  __shared__ Block blk[kWave];
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int32_t* src = idx + row * k;
  for (int j = lane; j < k; j += kWave) {
    const int s = src[j];
    row_s[j] = s;
    row_p[j] = s >= 0 ? s / ps : -1;
  }
  __syncthreads();
  const int per = (k + kWave - 1) / kWave;
  Block b{0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  int seg = 0;   // current page segment length
  for (int j = lane * per; j < min(k, (lane + 1) * per); ++j) {
    const int s = row_s[j];
    if (s < 0) continue;
    const int pg = row_p[j];
    if (b.cnt == 0) {
      b.first = s;
      b.pfirst = pg;
      b.runs = 1;
      b.pages = 1;
      seg = 1;
    } else {
      if (s != b.last + 1) ++b.runs;
      if (pg != b.plast) {
        if (b.pages == 1) b.head = seg;
        b.mx = max(b.mx, seg);
        ++b.pages;
        seg = 1;
      } else {
        ++seg;
      }
    }
    b.last = s;
    b.plast = pg;
    ++b.cnt;
  }
  if (b.cnt > 0) {
    if (b.pages == 1) b.head = seg;
    b.tail = seg;
    b.mx = max(b.mx, seg);
  }
  blk[lane] = b;
  __syncthreads();
  for (int w = 1; w < kWave; w <<= 1) {   // blocks [l, l+2w) from [l, l+w) and [l+w, l+2w)
    Block m;
    const bool act = (lane & (2 * w - 1)) == 0;
    if (act) m = merge(blk[lane], blk[lane + w]);
    __syncthreads();
    if (act) blk[lane] = m;
    __syncthreads();
  }
  if (lane == 0) {
    const Block r = blk[0];
    stats[row * 3 + 0] = r.pages;
    stats[row * 3 + 1] = r.runs;
    stats[row * 3 + 2] = r.mx;
  }
}

}  // namespace

hipError_t launch_gather_stats(const int32_t* idx, int32_t* stats, int64_t rows, int k, int page_size,
                               hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_stats_kernel, dim3((unsigned)rows), dim3(kWave), 0, st, idx, stats, rows, k, page_size);
  return hipGetLastError();
}

}  // namespace dsa
