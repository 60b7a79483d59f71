// Masked MHA mode of MLA for short prefills (the technical report's Inference
// Costs paragraph, forum translation Sec. 3; the analysis page's Fig. 3
// discussion and, for the two MLA forms, its MQA-mode discussion around
// Fig. 7).  Below a few thousand tokens the dense attention of MHA mode is
// cheaper than gathering 576-d latents per head group, so DSA is simulated
// there: every causal key is scored in MHA mode and the keys outside the
// row's top-k set are masked out of the softmax.
//
// Three kernels:
//   selection_mask   top-k index lists -> one bit per (row, key), stored
//                    [B, ceil(S/32), T] so a chunk's words for consecutive
//                    query rows are contiguous;
//   mha_decompress   per-head keys K_h = C W_UK[h]^T and values
//                    V_h = C W_UV[h]^T of the latent rows C (bf16 MFMA GEMM,
//                    LDS-staged, fp32 accumulation, bf16 out [B, H, rows, d]);
//   masked_mha       dense causal flash attention per (sequence, head,
//                    128 query rows), keys [K_h | rope] (rope dims of the
//                    latent row, shared by the heads), values V_h, the mask
//                    bits applied before the softmax.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Wave-uniform count of copies left in flight.
__device__ __forceinline__ void wait_vm_n(int n) {
  switch (n) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<1>(); break;
    case 2: wait_vm<2>(); break;
    case 3: wait_vm<3>(); break;
    case 4: wait_vm<4>(); break;
    case 5: wait_vm<5>(); break;
    case 6: wait_vm<6>(); break;
    case 7: wait_vm<7>(); break;
    default: wait_vm<8>(); break;
  }
}

// Swizzle of 16-byte pieces in rows of P pieces that are read 16 rows at a
// time (one piece per row, same logical piece): position = piece ^ swz, so
// the 16 reads of a ds_read_b128 pass hit 16 distinct 4-bank groups.
template <int P>
__device__ __forceinline__ int swz16(int r) { return (r / (16 / P)) % P; }

// ---------------------------------------------------------------- selection mask
constexpr int kMaskRows = 4;    // query rows per workgroup

__global__ void __launch_bounds__(256) selection_mask_kernel(MaskArgs a) {
  extern __shared__ uint32_t bits[];     // [kMaskRows][NC + 1]
  const int b = blockIdx.y;
  const int r0 = blockIdx.x * kMaskRows;   // first row of this block within the span
  const int ld = a.NC + 1;
  for (int e = threadIdx.x; e < kMaskRows * ld; e += 256) bits[e] = 0u;
  __syncthreads();
  const int nr = min(kMaskRows, a.rows - r0);
  for (int e = threadIdx.x; e < nr * a.k; e += 256) {
    const int r = e / a.k;
    const int s = a.idx[((int64_t)b * a.idx_rows_b + r0 + r) * a.k + e % a.k];
    const int n = min(a.pos0 + a.row0 + r0 + r + 1, a.S);    // keys s < n are causal
    if (s >= 0 && s < n) atomicOr(&bits[r * ld + (s >> 5)], 1u << (s & 31));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.NC * kMaskRows; e += 256) {
    const int c = e / kMaskRows, r = e % kMaskRows;
    if (r < nr) a.mask[((int64_t)b * a.NC + c) * a.T + a.row0 + r0 + r] = bits[r * ld + c];
  }
}

// ---------------------------------------------------------------- decompression GEMM
// out[s, n] = sum_c kv[s, c] * W[n, c] for one (sequence, head, matrix) and
// a tile of 128 rows s x TN columns n.  K (the compressed latent dims) runs
// in stages of 64, double-buffered in LDS by global_load_lds DMA.  Rows of a
// stage tile are 64 dims (8 pieces), piece p of row r at p ^ ((r / 2) % 8).
template <int TN>
struct DecCfg {
  static constexpr int kWN = TN >= 64 ? 2 : 1;        // waves along N
  static constexpr int kWM = 4 / kWN;                 // waves along M
  static constexpr int kMT = 128 / kWM / 32;          // 32-row blocks per wave
  static constexpr int kNT = TN / kWN / 32;           // 32-col blocks per wave
  static constexpr int kStageA = 128 * 64;            // elements
  static constexpr int kStageB = TN * 64;
  static constexpr int kStage = kStageA + kStageB;
  static constexpr int kDmaA = 128 * 8 / 64;          // 16 instructions
  static constexpr int kDmaB = TN * 8 / 64;
  static constexpr int kDma = kDmaA + kDmaB;
  static constexpr int kOutLd = TN + 8;               // epilogue staging row (elements)
  static constexpr int kSmem = 2 * kStage > 128 * kOutLd ? 2 * kStage : 128 * kOutLd;
  static_assert(kDma % 4 == 0, "DMA instructions must split evenly over 4 waves");
  static_assert(kMT * kWM * 32 == 128 && kNT * kWN * 32 == TN, "wave tiling");
};

__device__ __forceinline__ int dec_pos(int r, int p) { return r * 8 + (p ^ ((r >> 1) & 7)); }

template <int TN>
__global__ void __launch_bounds__(256, 2) mha_decompress_kernel(DecompArgs a) {
  using C = DecCfg<TN>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[C::kSmem];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int wm = wave / C::kWN, wn = wave % C::kWN;

  const int tiles_k = a.rows_w[0] / TN;                 // N tiles of the key matrix
  const int per_head = tiles_k + a.rows_w[1] / TN;
  const int h = blockIdx.y / per_head;
  int nt = blockIdx.y % per_head;
  const int which = nt < tiles_k ? 0 : 1;
  if (which) nt -= tiles_k;
  const int rows_w = a.rows_w[which];
  const int b = blockIdx.z;
  const int s0 = blockIdx.x * 128;
  const int n0 = nt * TN;

  const uint16_t* kvb = a.kv + (int64_t)b * a.S * a.Dk;
  const uint16_t* wb = a.w[which] + ((int64_t)h * rows_w + n0) * a.Dv;
  const int last = a.n_rows - 1;

  auto issue = [&](int kk, uint16_t* stage) {
    const int k0 = kk * 64;
#pragma unroll
    for (int jj = 0; jj < C::kDma / 4; ++jj) {
      const int j = jj * 4 + wave;
      if (j < C::kDmaA) {
        const int q = j * 64 + lane, r = q >> 3, pp = q & 7;
        const int s = min(s0 + r, last);
        dma_x4(kvb + (int64_t)s * a.Dk + k0 + 8 * (pp ^ ((r >> 1) & 7)), lds_addr(stage + j * 64 * 8));
      } else {
        const int q = (j - C::kDmaA) * 64 + lane, r = q >> 3, pp = q & 7;
        dma_x4(wb + (int64_t)r * a.Dv + k0 + 8 * (pp ^ ((r >> 1) & 7)),
               lds_addr(stage + C::kStageA + (j - C::kDmaA) * 64 * 8));
      }
    }
  };

  v16f acc[C::kMT][C::kNT];
#pragma unroll
  for (int i = 0; i < C::kMT; ++i)
#pragma unroll
    for (int j = 0; j < C::kNT; ++j) acc[i][j] = (v16f){};

  const int nk = a.Dv / 64;
  issue(0, smem);
  for (int kk = 0; kk < nk; ++kk) {
    uint16_t* cur = smem + (kk & 1) * C::kStage;
    wait_vm<0>();
    asm volatile("s_barrier" ::: "memory");
    if (kk + 1 < nk) issue(kk + 1, smem + ((kk + 1) & 1) * C::kStage);
    const uint16_t* sa = cur;
    const uint16_t* sb = cur + C::kStageA;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      v8bf av[C::kMT], bv[C::kNT];
#pragma unroll
      for (int i = 0; i < C::kMT; ++i) {
        const int r = 32 * (wm * C::kMT + i) + col;
        av[i] = *(const v8bf*)(sa + dec_pos(r, 2 * ks + half) * 8);
      }
#pragma unroll
      for (int j = 0; j < C::kNT; ++j) {
        const int r = 32 * (wn * C::kNT + j) + col;
        bv[j] = *(const v8bf*)(sb + dec_pos(r, 2 * ks + half) * 8);
      }
#pragma unroll
      for (int i = 0; i < C::kMT; ++i)
#pragma unroll
        for (int j = 0; j < C::kNT; ++j) acc[i][j] = mfma_bf16_32x32x16(av[i], bv[j], acc[i][j]);
    }
  }
  // Epilogue: bf16 tile through LDS, then 16-byte row stores.
  __syncthreads();
#pragma unroll
  for (int i = 0; i < C::kMT; ++i)
#pragma unroll
    for (int j = 0; j < C::kNT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 32 * (wm * C::kMT + i) + 8 * (e >> 2) + 4 * half + (e & 3);
        const int c = 32 * (wn * C::kNT + j) + col;
        smem[r * C::kOutLd + c] = (uint16_t)f32_to_bf16_rne(acc[i][j][e]);
      }
  __syncthreads();
  uint16_t* ob = a.out[which] + (((int64_t)b * a.H + h) * a.S_h) * rows_w + n0;
  constexpr int kPieces = TN / 8;
  for (int e = threadIdx.x; e < 128 * kPieces; e += 256) {
    const int r = e / kPieces, p = e % kPieces;
    if (s0 + r < a.n_rows)
      *(u32x4*)(ob + (int64_t)(s0 + r) * rows_w + 8 * p) = *(const u32x4*)(smem + r * C::kOutLd + 8 * p);
  }
}

// ---------------------------------------------------------------- masked MHA attention
// Workgroup: one (sequence b, head h, 128 query rows); wave w owns query
// rows t0 + 32w .. t0 + 32w + 31.  Keys run in chunks of 32 from s = 0 to
// the block's last position, through a three-deep ring of LDS tiles filled
// by DMA two chunks ahead.  A tile holds, for its 32 keys: the per-head key
// dims (DN), the rope dims of the latent rows (DR), the per-head values
// (DVH), and the 128 mask words of the block's query rows.  Per chunk and
// wave:
//   S^T[32 keys x 32 rows] = [K_h | rope] . Q^T    (A = keys from LDS, B = the
//                              wave's Q^T held in registers)
//   masked online softmax, lane-local (one query row per lane column)
//   O^T[DVH x 32 rows] += V^T . P^T                (A = V^T by transposed LDS
//                              reads, B = P^T straight from the S^T registers)
// The softmax reference of a row is raised only when a chunk's maximum
// exceeds it by more than kRefSlack (log2 units); O and the sum are then
// rescaled once.  Probabilities stay below 2^kRefSlack, far inside fp32 and
// bf16 range.
constexpr float kRefSlack = 16.0f;

template <int DN, int DR, int DVH>
struct MhaCfg {
  static constexpr int kPK = DN / 8, kPR = DR / 8, kPV = DVH / 8;     // pieces per row
  static constexpr int kKS = (DN + DR) / 16;                          // QK K steps
  static constexpr int kNT = DVH / 32;                                // O^T dim tiles
  static constexpr int kOffR = 32 * DN;                               // element offsets in a tile
  static constexpr int kOffV = kOffR + 32 * DR;
  static constexpr int kOffM = kOffV + 32 * DVH;
  static constexpr int kTileElems = kOffM + 2 * 128;                  // + 128 u32 mask words
  static constexpr int kDmaK = kPK / 2, kDmaR = kPR / 2, kDmaV = kPV / 2, kDmaM = 2;
  static constexpr int kDma = kDmaK + kDmaR + kDmaV + kDmaM;
  static_assert(kPK % 2 == 0 && kPR % 2 == 0 && kPV % 2 == 0, "tile rows must fill whole DMA instructions");
  static_assert(kPV == 4 || kPV == 16, "value head dim 32 or 128");
  static_assert(kPK <= 16 && kPR <= 16, "key rows of at most 128 dims per part");
  static_assert((kDma + 3) / 4 <= 8, "DMA instructions per wave");
};

// V part swizzle: the transposed reads of one pass cover 4 consecutive rows
// x 4 consecutive pieces; XOR with 4 * (r % 4) spreads them over 16 groups.
template <int PV>
__device__ __forceinline__ int swz_v(int r) { return PV == 16 ? 4 * (r & 3) : 0; }

// QK A operand of K step ks: logical piece 2 ks + half of key row `col`
// (per-head key dims first, then the rope dims).
template <int DN, int DR, int DVH>
__device__ __forceinline__ v8bf mha_load_a(const uint16_t* tile, int ks, int half, int col) {
  using C = MhaCfg<DN, DR, DVH>;
  const int p = 2 * ks + half;
  if (2 * ks < C::kPK) return *(const v8bf*)(tile + (col * C::kPK + (p ^ swz16<C::kPK>(col))) * 8);
  const int pr = p - C::kPK;
  return *(const v8bf*)(tile + C::kOffR + (col * C::kPR + (pr ^ swz16<C::kPR>(col))) * 8);
}

// S^T chain over K steps, the first three A operands already loaded.  The
// accumulator is a VGPR tuple (inline asm, next to the softmax that reads
// it); the wait states before its first VALU read are explicit.
template <int DN, int DR, int DVH>
__device__ __forceinline__ v16f mha_qk(const uint16_t* tile, v8bf (&abuf)[3], const v8bf (&qb)[(DN + DR) / 16],
                                       int half, int col) {
  using C = MhaCfg<DN, DR, DVH>;
  v16f st;
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks) {
    const v8bf cur = abuf[ks % 3];
    if (ks + 3 < C::kKS) abuf[ks % 3] = mha_load_a<DN, DR, DVH>(tile, ks + 3, half, col);
    if (ks == 0)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(st) : "v"(cur), "v"(qb[ks]));
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(st) : "v"(cur), "v"(qb[ks]));
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(st));
  return st;
}

// Copies per wave of one tile region of n DMA instructions: wave w issues
// instructions w, w + 4, ...
__host__ __device__ constexpr int dma_share(int n, int w) { return n > w ? (n - w + 3) / 4 : 0; }

template <int DN, int DR, int DVH>
__global__ void __launch_bounds__(256, 2) masked_mha_kernel(MhaArgs a) {
  using C = MhaCfg<DN, DR, DVH>;
  __shared__ __attribute__((aligned(16))) uint16_t tile0[C::kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t tile1[C::kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t tile2[C::kTileElems];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;

  // Work item: consecutive items of one XCD share a head (its K_h / V_h stay
  // in that XCD's L2); within a head the longest query blocks come first.
  const int n_items = gridDim.x;
  int w = blockIdx.x;
  if ((n_items & 7) == 0) w = (w & 7) * (n_items >> 3) + (w >> 3);
  const int ntq = (a.T + 127) / 128;
  const int bh = w / ntq;
  const int qt = ntq - 1 - w % ntq;
  const int b = bh / a.H, h = bh % a.H;
  const int t0 = qt * 128;
  const int t_last = min(t0 + 127, a.T - 1);
  const int p_last = a.pos0 + t_last;                   // < S
  const int nch = (p_last + 32) / 32;

  // This lane's query row and its causal key count.
  const int t = t0 + 32 * wave + col;
  const bool row_ok = t < a.T;
  const int n_keys = row_ok ? min(a.pos0 + t + 1, a.S) : 0;

  // Q^T operand (B of the QK product), kept in registers for the block.
  v8bf qb[C::kKS];
  {
    const uint16_t* qp = a.q + (((int64_t)b * a.T + min(t, a.T - 1)) * a.H + h) * (DN + DR) + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::kKS; ++ks) {
      v8bf v = *(const v8bf*)(qp + 16 * ks);
      if (!row_ok) v = (v8bf){};
      qb[ks] = v;
    }
  }
  wait_vm<0>();

  const uint16_t* khb = a.kh + ((int64_t)b * a.H + h) * a.S_h * DN;
  const uint16_t* vhb = a.vh + ((int64_t)b * a.H + h) * a.S_h * DVH;
  const uint16_t* kvb = a.kv + (int64_t)b * a.S * a.Dk + a.Dv;
  const uint32_t* mb = a.mask + (int64_t)b * a.NC * a.T;
  // This wave's DMA instructions per chunk (the same for every chunk).
  const int nd = dma_share(C::kDmaK, wave) + dma_share(C::kDmaR, wave) + dma_share(C::kDmaV, wave) +
                 dma_share(C::kDmaM, wave);

  // Rows past the block's last position are clamped to it (finite data,
  // masked out below).  Every copy takes a wave-uniform base in SGPRs and a
  // 32-bit byte offset per lane (a head's K_h / V_h block, a sequence's
  // latent cache and its mask are each below 4 GiB).  Wave w issues
  // instructions w, w + 4, ... of every region, so the addresses are
  // compile-time offsets from a few per-lane bases.
  auto gather = [&](int c, uint16_t* tl) {
    const int s0 = 32 * c;
#pragma unroll
    for (int i = 0; i < (C::kDmaK + 3) / 4; ++i) {
      const int j = wave + 4 * i;
      if ((C::kDmaK % 4) == 0 || j < C::kDmaK) {
        const int q = j * 64 + lane, r = q / C::kPK, pp = q % C::kPK;
        const uint32_t s = (uint32_t)min(s0 + r, p_last);
        dma_x4_s((s * DN + 8 * (pp ^ swz16<C::kPK>(r))) * 2u, khb, lds_addr(tl + j * 512));
      }
    }
#pragma unroll
    for (int i = 0; i < (C::kDmaR + 3) / 4; ++i) {
      const int j = wave + 4 * i;
      if ((C::kDmaR % 4) == 0 || j < C::kDmaR) {
        const int q = j * 64 + lane, r = q / C::kPR, pp = q % C::kPR;
        const uint32_t s = (uint32_t)min(s0 + r, p_last);
        dma_x4_s((s * (uint32_t)a.Dk + 8 * (pp ^ swz16<C::kPR>(r))) * 2u, kvb, lds_addr(tl + C::kOffR + j * 512));
      }
    }
#pragma unroll
    for (int i = 0; i < (C::kDmaV + 3) / 4; ++i) {
      const int j = wave + 4 * i;
      if ((C::kDmaV % 4) == 0 || j < C::kDmaV) {
        const int q = j * 64 + lane, r = q / C::kPV, pp = q % C::kPV;
        const uint32_t s = (uint32_t)min(s0 + r, p_last);
        dma_x4_s((s * DVH + 8 * (pp ^ swz_v<C::kPV>(r))) * 2u, vhb, lds_addr(tl + C::kOffV + j * 512));
      }
    }
    if (wave < C::kDmaM) {
      const uint32_t tq = (uint32_t)min(t0 + 64 * wave + lane, a.T - 1);
      dma_x1_s(((uint32_t)c * (uint32_t)a.T + tq) * 4u, mb, lds_addr(tl + C::kOffM + wave * 128));
    }
  };

  // Transposed V^T operand reads (the lane mapping of the sparse MLA
  // kernel): lane group g = lane / 16 covers rows 4 * (g / 2) + jl / 4 of a
  // 4-row block and dims 16 * (g % 2) + 4 * (jl % 4) .. + 3 of a 32-dim tile.
  const int g = lane >> 4, jl = lane & 15;
  const int vrow = 4 * (g >> 1) + (jl >> 2);
  const int vpiece = 2 * (g & 1) + ((jl & 3) >> 1);
  const int vsub = 4 * (jl & 1);
  // Rows vrow and vrow + 8 (+ 16 per K step) share r % 4, so the swizzle
  // turns dim tile ti into piece group ti ^ (vrow % 4) for every read.
  const int vswz = swz_v<C::kPV>(vrow) >> 2;
  const int v_lo = C::kOffV + vrow * C::kPV * 8 + vpiece * 8 + vsub;
  const int v_hi = v_lo + 8 * C::kPV * 8;
  constexpr int kM = 2 * C::kNT;             // PV MFMAs per chunk
  constexpr int kLookV = kM < 4 ? kM : 4;    // PV operands in flight
  auto load_v = [&](const uint16_t* tl, int m) {
    const int ti = m >> 1, kk = m & 1;
    const int off = 16 * kk * C::kPV * 8 + 32 * (ti ^ vswz);
    const v4bf lo = lds_read_tr16(tl + v_lo + off);
    const v4bf hi = lds_read_tr16(tl + v_hi + off);
    return (v8bf)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  v16f o[C::kNT];
#pragma unroll
  for (int i = 0; i < C::kNT; ++i) o[i] = (v16f){};
  float m_ref = -INFINITY, l_sum = 0.f;
  const float zscale = a.sm_scale * kLog2e;

  auto attend = [&](int c, const uint16_t* tl) {
    // The mask word and the first QK operands are read together.
    uint32_t word = ((const uint32_t*)(tl + C::kOffM))[32 * wave + col];
    v8bf abuf[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) abuf[j] = mha_load_a<DN, DR, DVH>(tl, j, half, col);
    const int nv = n_keys - 32 * c;                     // causal keys of this chunk
    if (nv < 32) word &= nv <= 0 ? 0u : ((1u << nv) - 1u);
    if (__builtin_amdgcn_ballot_w64(word != 0u) == 0) return;   // wave-uniform
    const v16f st = mha_qk<DN, DR, DVH>(tl, abuf, qb, half, col);
    // V^T operands of the first PV MFMAs, in flight during the softmax.
    v8bf vbuf[kLookV];
#pragma unroll
    for (int j = 0; j < kLookV; ++j) vbuf[j] = load_v(tl, j);
    float z[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) z[j] = st[j];
    if (__builtin_amdgcn_ballot_w64(word != 0xFFFFFFFFu) != 0) {
      const uint32_t vh = word >> (4 * half);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        // keep = all ones if key row 8 (j / 4) + j % 4 (+ 4 half) is selected
        const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)vh, 8 * (j >> 2) + (j & 3), 1);
        z[j] = __uint_as_float((__float_as_uint(z[j]) & keep) | (0xFF800000u & ~keep));
      }
    }
    float mx = z[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = __builtin_fmaxf(mx, z[j]);
    mx = max_halves(mx) * zscale;                       // zscale > 0
    const bool raise = mx > m_ref + kRefSlack;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float m_new = raise ? mx : m_ref;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
#pragma unroll
      for (int i = 0; i < C::kNT; ++i) o[i] *= alpha;
      l_sum *= alpha;
      m_ref = m_new;
    }
    const float nref = m_ref == -INFINITY ? 0.f : -m_ref;
    v8bf pb[2];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float pj = __builtin_amdgcn_exp2f(__builtin_fmaf(z[j], zscale, nref));
      l_sum += pj;
      pb[j >> 3][j & 7] = (__bf16)pj;
    }
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      const v8bf cur = vbuf[m % kLookV];
      if (m + kLookV < kM) vbuf[m % kLookV] = load_v(tl, m + kLookV);
      o[m >> 1] = mfma_bf16_32x32x16(cur, pb[m & 1], o[m >> 1]);
    }
  };

  // Chunk c lives in tile c % 3; its DMA is issued after the barrier of
  // chunk c - 2, so each wave waits for its own copies of chunk c with chunk
  // c + 1's still in flight, then the barrier publishes the tile.
  auto step = [&](int c, const uint16_t* cur, uint16_t* fill) {
    if (c + 1 < nch) wait_vm_n(nd); else wait_vm<0>();
    asm volatile("s_barrier" ::: "memory");
    if (c + 2 < nch) gather(c + 2, fill);
    attend(c, cur);
  };
  gather(0, tile0);
  if (nch > 1) gather(1, tile1);
  for (int c = 0; c < nch; c += 3) {
    step(c, tile0, tile2);
    if (c + 1 >= nch) break;
    step(c + 1, tile1, tile0);
    if (c + 2 >= nch) break;
    step(c + 2, tile2, tile1);
  }

  // Epilogue: normalise and store (4 consecutive dims per 8-byte store).
  const float l_tot = sum_halves(l_sum);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* op = a.out + (((int64_t)b * a.T + t) * a.H + h) * DVH;
#pragma unroll
  for (int ti = 0; ti < C::kNT; ++ti)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * ti + 8 * g4 + 4 * half;
      uint2 v;
      v.x = pack_bf16x2(o[ti][4 * g4 + 0] * inv, o[ti][4 * g4 + 1] * inv);
      v.y = pack_bf16x2(o[ti][4 * g4 + 2] * inv, o[ti][4 * g4 + 3] * inv);
      *(uint2*)(op + d0) = v;
    }
  if (a.lse && half == 0)
    a.lse[((int64_t)b * a.T + t) * a.H + h] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int DN, int DR, int DVH>
hipError_t launch_mha_cfg(const MhaArgs& a, hipStream_t st) {
  const int64_t items = (int64_t)a.B * a.H * ((a.T + 127) / 128);
  hipLaunchKernelGGL((masked_mha_kernel<DN, DR, DVH>), dim3((unsigned)items), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

bool mha_dims_supported(int dn, int dr, int dvh, int Dv) {
  return (dn == 128 && dr == 64 && dvh == 128 && Dv % 64 == 0) || (dn == 32 && dr == 16 && dvh == 32 && Dv % 64 == 0);
}

hipError_t launch_selection_mask(const MaskArgs& a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  const size_t smem = (size_t)kMaskRows * (a.NC + 1) * sizeof(uint32_t);
  hipLaunchKernelGGL(selection_mask_kernel, dim3((unsigned)((a.rows + kMaskRows - 1) / kMaskRows), (unsigned)a.B),
                     dim3(256), smem, st, a);
  return hipGetLastError();
}

hipError_t launch_mha_decompress(const DecompArgs& a, hipStream_t st) {
  if (a.n_rows <= 0) return hipSuccess;
  const bool wide = a.rows_w[0] % 128 == 0 && a.rows_w[1] % 128 == 0;
  const int tn = wide ? 128 : 32;
  const dim3 grid((unsigned)((a.n_rows + 127) / 128), (unsigned)(a.H * (a.rows_w[0] / tn + a.rows_w[1] / tn)),
                  (unsigned)a.B);
  if (wide) hipLaunchKernelGGL(mha_decompress_kernel<128>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(mha_decompress_kernel<32>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_masked_mha(const MhaArgs& a, int dn, int dr, int dvh, hipStream_t st) {
  if (dn == 128 && dr == 64 && dvh == 128) return launch_mha_cfg<128, 64, 128>(a, st);
  if (dn == 32 && dr == 16 && dvh == 32) return launch_mha_cfg<32, 16, 32>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace dsa
