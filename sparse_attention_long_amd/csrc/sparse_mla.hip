// Sparse MLA attention in MQA mode over the selected latent rows (page
// "DeepSeek-V3.2: sparse attention, scaled RL and synthetic agent
// environments", Sec. 1.1 Eq. (2) and the MQA-mode discussion around Fig. 7;
// softmax renormalised over the selected set, Sec. 5.2 Eq. (19)).
//
// For every query row, all H heads attend over the same gathered rows c_s
// (keys: all Dk dims; values: the first Dv dims), so each gathered row is
// read from memory once per query and used by every head.
//
// Work shape (gfx950): one workgroup per (query row, split of the selected
// slots); wave w owns heads [32w, 32w+32).  Rows are gathered 32 at a time
// into a double-buffered LDS tile.  Per chunk and wave:
//   S^T[32 rows x 32 heads] = C[32 x Dk] . Q^T[Dk x 32]   (v_mfma_f32_32x32x16_bf16,
//        A = C from LDS, B = the wave's Q^T kept in registers for the whole row)
//   online softmax per head (lane-local: the S^T layout puts one head per lane)
//   O^T[Dv x 32 heads] += V^T[Dv x 32 rows] . P^T[32 rows x 32 heads]
// The P^T operand is the softmax output in the very registers the S^T MFMA
// produced (the K order of the PV product is permuted to match the S^T row
// order; V^T is read from LDS in that same order), so P never goes through
// LDS.  Each head's softmax reference is the maximum logit of its first
// chunk and is not raised afterwards: fp32/bf16 keep 8 exponent bits, so
// probabilities up to 2^64 above that reference are exact enough and cannot
// overflow.  Only if a later logit exceeds the reference by more than 64
// (log2 units) is the row recomputed once with the true maximum as the
// reference.  No O rescale is ever needed, which keeps the 32x512 fp32
// accumulator of each wave in the AGPR file without spills.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kChunk = 32;             // gathered rows per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRefHeadroom = 64.0f;  // log2 units a logit may exceed the reference by
constexpr int kMaxSlots = 2048;

template <int DK, int DV, int NW>
struct Cfg {
  static constexpr int kKS = DK / 16;            // QK K steps
  static constexpr int kKSL = kKS / 2;           // K steps whose Q^T operand lives in LDS
  static constexpr int kKSR = kKS - kKSL;        // K steps whose Q^T operand lives in registers
  static constexpr int kHeads = NW * 32;
  static constexpr int kNT = DV / 32;            // O^T dim tiles
  static constexpr int kRS = DK + 8;             // LDS row stride (bf16): +16 B de-aligns banks
  static constexpr int kPieces = DK / 8;         // 16-byte pieces of data per row
  static constexpr int kSlotsRow = kRS / 8;      // 16-byte LDS slots per row (last one is padding)
  static constexpr int kSlots = kChunk * kSlotsRow;
  static constexpr int kThreads = NW * kWave;
  static constexpr int kDmaIters = (kSlots + kThreads - 1) / kThreads;
  static constexpr int kTileElems = kSlots * 8;
  static constexpr int kQElems = kKSL * 2 * kHeads * 8;   // Q^T part: [ks][half][head][8]
};

// Gather the 32 rows of chunk c straight into an LDS tile with
// global_load_lds_dwordx4: each wave instruction fills 64 consecutive
// 16-byte LDS slots, lane l filling slot base + l from the global row piece
// that belongs there.  Padding slots are skipped; an invalid row index reads
// row 0 instead (finite data, masked out of the softmax later).
template <int DK, int DV, int NW>
__device__ __forceinline__ void gather_dma(uint16_t* tile, const uint16_t* kvb, const int32_t* sidx_c) {
  using C = Cfg<DK, DV, NW>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < C::kDmaIters; ++u) {
    const int base = (u * NW + wave) * kWave;
    const int q = base + lane;
    const int r = q / C::kSlotsRow, p = q % C::kSlotsRow;
    if (q < C::kSlots && p < C::kPieces) {
      const int s = max(sidx_c[r], 0);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(kvb + (int64_t)s * DK + 8 * p),
          (__attribute__((address_space(3))) void*)(tile + base * 8), 16, 0, 0);
    }
  }
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int DK, int DV, int NW>
struct RowState {
  v16f o[Cfg<DK, DV, NW>::kNT];
  float m_ref;   // softmax reference of this lane's head (log2 units), fixed during a pass
  float m_seen;  // largest logit seen (log2 units)
  float l_sum;   // this half's share of the softmax denominator
};

// One chunk of 32 gathered rows: S^T = C.Q^T, softmax weights against the
// fixed reference, O^T += V^T.P^T.
template <int DK, int DV, int NW>
__device__ __forceinline__ void attend_chunk(const uint16_t* tb, const int32_t* sidx_c, const uint16_t* qlds,
                                             const v8bf (&qb)[Cfg<DK, DV, NW>::kKSR], float zscale,
                                             RowState<DK, DV, NW>& rs) {
  using C = Cfg<DK, DV, NW>;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, col = lane & 31;
  // ---- S^T = C . Q^T
  v16f st = {};
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int ks = 0; ks < C::kKSL; ++ks) {
    const v8bf av = *(const v8bf*)(tb + col * C::kRS + 16 * ks + 8 * half);
    const v8bf bv = *(const v8bf*)(qlds + ((ks * 2 + half) * C::kHeads + wave * 32 + col) * 8);
    st = mfma_bf16_32x32x16(av, bv, st);
  }
#pragma unroll
  for (int ks = 0; ks < C::kKSR; ++ks) {
    const v8bf av = *(const v8bf*)(tb + col * C::kRS + 16 * (C::kKSL + ks) + 8 * half);
    st = mfma_bf16_32x32x16(av, qb[ks], st);
  }
  // ---- mask, scale, chunk max
  float z[16];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = 8 * (j >> 2) + 4 * half + (j & 3);
    z[j] = sidx_c[r] >= 0 ? st[j] * zscale : -INFINITY;
    mx = fmaxf(mx, z[j]);
  }
  mx = max_halves(mx);
  if (rs.m_ref == -INFINITY) rs.m_ref = mx;
  rs.m_seen = fmaxf(rs.m_seen, mx);
  // ---- probabilities, packed as the P^T operand (K order = S^T row order)
  v8bf pb[2];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float pj = exp2f(z[j] - rs.m_ref);
    rs.l_sum += pj;
    pb[j >> 3][j & 7] = (__bf16)pj;
  }
  // ---- O^T += V^T . P^T ; K index k of step kk is row 16*kk + 8*((k%8)/4) + 4*(k/8) + k%4
#pragma unroll
  for (int t = 0; t < C::kNT; ++t) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      v8bf vv;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int r = 16 * kk + 8 * (jj >> 2) + 4 * half + (jj & 3);
        vv[jj] = __builtin_bit_cast(__bf16, tb[r * C::kRS + 32 * t + col]);
      }
      rs.o[t] = mfma_bf16_32x32x16(vv, pb[kk], rs.o[t]);
    }
  }
}

template <int DK, int DV, int NW>
__global__ void __launch_bounds__(NW * kWave, 1) sparse_mla_kernel(AttnArgs a) {
  using C = Cfg<DK, DV, NW>;
  __shared__ __attribute__((aligned(16))) uint16_t tile0[C::kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t tile1[C::kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t qlds[C::kQElems];
  __shared__ int32_t sidx[kMaxSlots];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int rowid = blockIdx.x / a.nsplit;       // b * rows + i
  const int sp = blockIdx.x % a.nsplit;
  const int b = rowid / a.rows;
  const int i = rowid % a.rows;
  const int64_t qrow = (int64_t)b * a.qrows_b + i;

  // Slots of this split, in whole chunks.
  const int per_split = ((a.k + a.nsplit - 1) / a.nsplit + kChunk - 1) / kChunk * kChunk;
  const int slot0 = sp * per_split;
  const int nslots = max(0, min(per_split, a.k - slot0));
  const int nchunks = (nslots + kChunk - 1) / kChunk;

  for (int j = threadIdx.x; j < nchunks * kChunk; j += C::kThreads) {
    int v = -1;
    if (j < nslots) {
      v = a.idx[((int64_t)b * a.idx_rows_b + i) * a.k + slot0 + j];
      if (v < 0 || v >= a.S) v = -1;
    }
    sidx[j] = v;
  }

  // Q^T operand for the whole row: K steps [0, kKSL) of all heads in LDS,
  // laid out [ks][half][head][8] so a wave's 16-byte reads are consecutive;
  // K steps [kKSL, kKS) of this wave's 32 heads in registers.
  for (int pc = threadIdx.x; pc < C::kKSL * 2 * C::kHeads; pc += C::kThreads) {
    const int hh = pc % C::kHeads, kh = pc / C::kHeads;   // kh = ks * 2 + half
    v8bf v = {};
    if (hh < a.H) v = *(const v8bf*)(a.q + (qrow * a.H + hh) * DK + 8 * kh);
    *(v8bf*)(qlds + pc * 8) = v;
  }
  const int h = wave * 32 + col;
  v8bf qb[C::kKSR];
  {
    const uint16_t* qp = a.q + (qrow * a.H + min(h, a.H - 1)) * DK + 16 * C::kKSL + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::kKSR; ++ks) {
      v8bf v = *(const v8bf*)(qp + 16 * ks);
      if (h >= a.H) v = (v8bf){};
      qb[ks] = v;
    }
  }
  __syncthreads();

  const uint16_t* kvb = a.kv + (int64_t)b * a.S * DK;
  RowState<DK, DV, NW> rs;
  rs.m_ref = -INFINITY;
  rs.m_seen = -INFINITY;
  const float zscale = a.sm_scale * kLog2e;
  __shared__ int redo;

  auto chunk_valid = [&](int c) {
    return __builtin_amdgcn_ballot_w64(lane < kChunk && sidx[c * kChunk + (lane & 31)] >= 0) != 0;
  };
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int t = 0; t < C::kNT; ++t) rs.o[t] = (v16f){};
    rs.l_sum = 0.f;
    if (threadIdx.x == 0) redo = 0;
    // Double buffering: chunk c is read from tile(c%2) while chunk c+1 is
    // DMA'd into the other tile; one barrier per chunk.
    if (nchunks > 0) gather_dma<DK, DV, NW>(tile0, kvb, sidx);
    wait_dma();
    __syncthreads();
    for (int c = 0; c < nchunks; c += 2) {
      if (c + 1 < nchunks) gather_dma<DK, DV, NW>(tile1, kvb, sidx + (c + 1) * kChunk);
      if (chunk_valid(c)) attend_chunk<DK, DV, NW>(tile0, sidx + c * kChunk, qlds, qb, zscale, rs);
      wait_dma();
      __syncthreads();
      if (c + 1 >= nchunks) break;
      if (c + 2 < nchunks) gather_dma<DK, DV, NW>(tile0, kvb, sidx + (c + 2) * kChunk);
      if (chunk_valid(c + 1)) attend_chunk<DK, DV, NW>(tile1, sidx + (c + 1) * kChunk, qlds, qb, zscale, rs);
      wait_dma();
      __syncthreads();
    }
    // A logit far above its head's reference: redo the row with the true max.
    if (rs.m_seen > rs.m_ref + kRefHeadroom) redo = 1;
    __syncthreads();
    if (!redo) break;
    rs.m_ref = rs.m_seen;
    __syncthreads();
  }

  // ---- epilogue
  const float l_tot = sum_halves(rs.l_sum);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (rs.m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
  if (h < a.H) {
    if (a.nsplit == 1) {
      uint16_t* op = a.out + (qrow * a.H + h) * DV;
#pragma unroll
      for (int t = 0; t < C::kNT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * t + 8 * g + 4 * half;
          uint2 pk;
          pk.x = pack_bf16x2(rs.o[t][4 * g + 0] * inv, rs.o[t][4 * g + 1] * inv);
          pk.y = pack_bf16x2(rs.o[t][4 * g + 2] * inv, rs.o[t][4 * g + 3] * inv);
          *(uint2*)(op + d) = pk;
        }
      if (a.lse && half == 0) a.lse[qrow * a.H + h] = lse_v;
    } else {
      float* pp = a.part_o + (((int64_t)rowid * a.nsplit + sp) * a.H + h) * DV;
#pragma unroll
      for (int t = 0; t < C::kNT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * t + 8 * g + 4 * half;
          float4 v = {rs.o[t][4 * g] * inv, rs.o[t][4 * g + 1] * inv, rs.o[t][4 * g + 2] * inv,
                      rs.o[t][4 * g + 3] * inv};
          *(float4*)(pp + d) = v;
        }
      if (half == 0) a.part_lse[((int64_t)rowid * a.nsplit + sp) * a.H + h] = lse_v;
    }
  }
}

// Merge split partials: lse = log sum_j exp(lse_j), o = sum_j exp(lse_j - lse) o_j.
template <int DV>
__global__ void __launch_bounds__(DV / 4) mla_combine_kernel(AttnArgs a) {
  const int rowid = blockIdx.x / a.H;
  const int h = blockIdx.x % a.H;
  const int b = rowid / a.rows, i = rowid % a.rows;
  const int64_t qrow = (int64_t)b * a.qrows_b + i;
  const float* pl = a.part_lse + (int64_t)rowid * a.nsplit * a.H + h;
  float mx = -INFINITY;
  for (int j = 0; j < a.nsplit; ++j) mx = fmaxf(mx, pl[(int64_t)j * a.H]);
  float den = 0.f;
  if (mx > -INFINITY)
    for (int j = 0; j < a.nsplit; ++j) den += __expf(pl[(int64_t)j * a.H] - mx);
  const float lse = mx > -INFINITY ? mx + __logf(den) : -INFINITY;
  const int d = threadIdx.x * 4;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  if (mx > -INFINITY) {
    for (int j = 0; j < a.nsplit; ++j) {
      const float lj = pl[(int64_t)j * a.H];
      if (lj == -INFINITY) continue;
      const float wj = __expf(lj - lse);
      const float4 v = *(const float4*)(a.part_o + (((int64_t)rowid * a.nsplit + j) * a.H + h) * DV + d);
      acc.x += wj * v.x; acc.y += wj * v.y; acc.z += wj * v.z; acc.w += wj * v.w;
    }
  }
  uint2 pk;
  pk.x = pack_bf16x2(acc.x, acc.y);
  pk.y = pack_bf16x2(acc.z, acc.w);
  *(uint2*)(a.out + (qrow * a.H + h) * DV + d) = pk;
  if (a.lse && threadIdx.x == 0) a.lse[qrow * a.H + h] = lse;
}

template <int DK, int DV, int NW>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)(a.B * a.rows * a.nsplit);
  hipLaunchKernelGGL((sparse_mla_kernel<DK, DV, NW>), dim3(grid), dim3(NW * kWave), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL((mla_combine_kernel<DV>), dim3((unsigned)(a.B * a.rows * a.H)), dim3(DV / 4), 0, st, a);
  return hipGetLastError();
}

}  // namespace

bool attn_dims_supported(int H, int Dk, int Dv) {
  if (Dk == 576 && Dv == 512) return H >= 1 && H <= 128;
  if (Dk == 80 && Dv == 64) return H >= 1 && H <= 32;
  return false;
}

hipError_t launch_sparse_mla(const AttnArgs& a, hipStream_t st) {
  if (a.rows <= 0 || a.B <= 0) return hipSuccess;
  if (a.Dk == 576 && a.Dv == 512) return launch_cfg<576, 512, 4>(a, st);
  if (a.Dk == 80 && a.Dv == 64) return launch_cfg<80, 64, 1>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace dsa
