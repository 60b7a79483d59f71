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
// into a three-deep ring of LDS tiles by global_load_lds DMA, two chunks
// ahead.  Per chunk and wave:
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
//
// A wave runs one chunk's phases back to back (gather issue, QK, softmax,
// PV), so the non-MFMA phases are kept short: the S^T chain accumulates in
// VGPRs (next to the softmax that reads it, not in the AGPR file next to
// O^T), the softmax folds scale and reference into one fma per logit and
// masks only a row's last chunk, and a row copy costs one lane read and one
// VALU op (scalar sequence base + 32-bit offset).
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kChunk = 32;             // gathered rows per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRefHeadroom = 64.0f;  // log2 units a logit may exceed the reference by
constexpr int kMaxSlots = 2048;
constexpr int kMaxSplits = 16;        // slot splits per row (the split rule caps them)
constexpr int kLookA = 3;              // QK operand prefetch depth (K steps)
constexpr int kLookV = 4;              // PV operand prefetch depth (MFMAs)

// LDS tile of one chunk (32 gathered rows), in 16-byte pieces:
//  part A: the value dims [0, Dv) of every row, row stride RA = PA + padA
//          pieces, piece p of row r stored at position p ^ ((r / 4) % 4);
//  part B: the remaining (rope) dims [Dv, Dk), PB pieces per row, piece p of
//          row r stored at p ^ (r % PB).
// With RA = 68 (1088 B, 272 dwords = 16 mod 64 banks) both the QK operand
// reads (16 rows x 16 B per pass) and the PV transposed reads (4 rows x 64 B
// per pass) touch 64 distinct banks.
template <int DK, int DV, int NW>
struct Cfg {
  static constexpr int kKS = DK / 16;            // QK K steps
  static constexpr int kNT = DV / 32;            // O^T dim tiles
  static constexpr int kPA = DV / 8;             // pieces of part A per row
  static constexpr int kPB = (DK - DV) / 8;      // pieces of part B per row
  static constexpr int kRA = kPA == 64 ? 68 : kPA;   // part A row stride (pieces)
  static constexpr int kBaseB = kChunk * kRA;    // first piece of part B
  static constexpr int kTilePieces = kBaseB + kChunk * kPB;
  static constexpr int kTileElems = kTilePieces * 8;
  static constexpr int kThreads = NW * kWave;
  // DMA instructions per chunk: one per row of part A when a row is exactly
  // one wave's 64 pieces, else 64 consecutive pieces each; then part B.
  static constexpr bool kRowDma = kPA == 64;
  static constexpr int kDmaA = kRowDma ? kChunk : kChunk * kPA / kWave;
  static constexpr int kDmaB = kChunk * kPB / kWave;
  static constexpr int kDma = kDmaA + kDmaB;
  static_assert(kPA % 4 == 0 && (kChunk * kPA) % kWave == 0 && (kChunk * kPB) % kWave == 0, "tile shape");
  static_assert((kPB & (kPB - 1)) == 0, "part B width must be a power of two");
  static_assert(kDma % NW == 0, "DMA instructions must split evenly over waves");
};

__device__ __forceinline__ int swz_a(int r) { return (r >> 2) & 3; }

// Position (in elements) of logical piece p of row r.
template <int DK, int DV, int NW>
__device__ __forceinline__ int piece_pos(int r, int p) {
  using C = Cfg<DK, DV, NW>;
  if (p < C::kPA) return (r * C::kRA + (p ^ swz_a(r))) * 8;
  const int pb = p - C::kPA;
  return (C::kBaseB + r * C::kPB + (pb ^ (r & (C::kPB - 1)))) * 8;
}

// Gather one chunk's rows into a tile with global_load_lds_dwordx4 (issued
// from inline asm, see dma_x4), for the shapes whose rows are not one wave
// instruction long: each wave instruction fills 64 consecutive 16-byte LDS
// pieces, lane l filling piece base + l from the global row piece that
// belongs there, with a 64-bit address per lane.  Instruction j goes to wave
// j % NW, so every wave issues kDma / NW instructions.  An invalid row index
// reads row 0 (finite data, masked out of the softmax).
template <int DK, int DV, int NW>
struct ChunkGather {
  using C = Cfg<DK, DV, NW>;
  static_assert(!C::kRowDma, "row-sized shapes use RowGather");
  uint16_t* tile;
  const uint16_t* kvb;
  int row_of_lane;    // lane j < 32 holds the chunk's j-th row index (or < 0)
  int wave;

  __device__ __forceinline__ void init(uint16_t* t, const uint16_t* kv, int rol) {
    tile = t;
    kvb = kv;
    row_of_lane = max(rol, 0);
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  }
  __device__ __forceinline__ void issue(int jj) const {
    const int lane = threadIdx.x & 63;
    const int j = jj * NW + wave;   // wave-uniform instruction index
    if (j < C::kDmaA) {
      const int q = j * kWave + lane;             // piece of the contiguous part A
      const int r = q / C::kPA, pp = q % C::kPA;
      const int s = __shfl(row_of_lane, r, kWave);
      dma_x4(kvb + (int64_t)s * DK + 8 * (pp ^ swz_a(r)), lds_addr(tile + j * kWave * 8));
    } else {
      const int q = (j - C::kDmaA) * kWave + lane;  // piece of part B
      const int r = q / C::kPB, pp = q % C::kPB;
      const int s = __shfl(row_of_lane, r, kWave);
      dma_x4(kvb + (int64_t)s * DK + 8 * (C::kPA + (pp ^ (r & (C::kPB - 1)))),
             lds_addr(tile + (C::kBaseB + (j - C::kDmaA) * kWave) * 8));
    }
  }
  __device__ __forceinline__ void issue_all() const {
#pragma unroll
    for (int jj = 0; jj < C::kDma / NW; ++jj) issue(jj);
  }
};

// Gather for the shapes whose part-A rows are exactly one wave instruction
// (Dv = 512) with 4 waves.  Wave w copies rows j = 4*jj + w (jj < 8) of part
// A, whose piece swizzle is jj % 4, and the part-B block of rows 8w .. 8w+7.
// Dense caches (K64 false): every copy takes the sequence's cache base as
// its scalar address and a 32-bit per-lane byte offset (a sequence's latent
// cache is below 4 GiB), so a row copy costs one lane read and one VALU op.
// Page pools (K64 true) may exceed 4 GiB: a row copy reads the row's 64-bit
// address into SGPRs (two lane reads) and part B uses 64-bit lane addresses.
template <int DK, int DV, int NW, bool K64>
struct RowGather {
  using C = Cfg<DK, DV, NW>;
  static_assert(C::kRowDma && NW == 4 && C::kDmaA == kChunk && C::kDmaB == NW, "row gather shape");
  uint32_t off_a;   // lane j < 32: byte offset of chunk row j (low half of it for K64)
  uint32_t off_ah;  // K64: high half
  uint64_t off_b;   // byte offset of this lane's part-B piece
  uint32_t lane16;  // 16 * lane

  // Chunk row whose index lane `lane` must supply for part B.
  __device__ __forceinline__ static int row_b(int wave, int lane) { return (wave * kWave + lane) / C::kPB; }

  __device__ __forceinline__ void init(int ra, int rb, int wave) {
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));   // keep the per-lane terms here, do not hoist them
    lane16 = 16u * (uint32_t)lane;
    const uint64_t oa = (uint64_t)max(ra, 0) * (uint64_t)(DK * 2);
    off_a = (uint32_t)oa;
    off_ah = (uint32_t)(oa >> 32);
    const int q = wave * kWave + lane;
    const int r = q / C::kPB, pp = q % C::kPB;
    off_b = (uint64_t)max(rb, 0) * (uint64_t)(DK * 2) + 16u * (uint32_t)(C::kPA + (pp ^ (r & (C::kPB - 1))));
  }
  static constexpr int kPerWave = C::kDmaA / NW + 1;   // copy instructions per wave and chunk
  // Copy instruction jj (< kPerWave) of this wave: part-A row jj * NW + wave,
  // or (jj = kPerWave - 1) the wave's part-B block.
  __device__ __forceinline__ void issue(int jj, uint16_t* tile, const uint16_t* kvb, int wave) const {
    const uint32_t t0 = lds_addr(tile);
    if (jj < C::kDmaA / NW) {
      const int j = jj * NW + wave;
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)off_a, j);
      if constexpr (K64) {
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)off_ah, j);
        const uint8_t* rowp = (const uint8_t*)kvb + (((uint64_t)hi << 32) | lo);
        dma_x4_s(lane16 ^ (16u * (uint32_t)(jj & 3)), rowp, t0 + (uint32_t)j * (C::kRA * 16));
      } else {
        dma_x4_s((lane16 ^ (16u * (uint32_t)(jj & 3))) + lo, kvb, t0 + (uint32_t)j * (C::kRA * 16));
      }
    } else if constexpr (K64) {
      dma_x4((const uint8_t*)kvb + off_b, t0 + (uint32_t)(C::kBaseB + wave * kWave) * 16u);
    } else {
      dma_x4_s((uint32_t)off_b, kvb, t0 + (uint32_t)(C::kBaseB + wave * kWave) * 16u);
    }
  }
  // All of a wave's copies for one chunk.  Dense caches: the lane offsets
  // and LDS targets are formed first and the nine copies then go out from
  // one asm block that sets M0 before each, so the copies do not wait on
  // one another's address arithmetic (the same copies in the same order as
  // issue(0..kPerWave-1)).
  __device__ __forceinline__ void issue_all(uint16_t* tile, const uint16_t* kvb, int wave) const {
    if constexpr (!K64) {
      static_assert(kPerWave == 9, "eight part-A rows and one part-B block per wave");
      const uint32_t t0 = lds_addr(tile);
      uint32_t vo[8], la[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = jj * NW + wave;
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)off_a, j);
        vo[jj] = (lane16 ^ (16u * (uint32_t)(jj & 3))) + lo;
        la[jj] = t0 + (uint32_t)j * (C::kRA * 16);
      }
      const uint32_t lb = t0 + (uint32_t)(C::kBaseB + wave * kWave) * 16u;
      uint32_t saved;
      asm volatile(
          "s_mov_b32 %0, m0\n\t"
          "s_mov_b32 m0, %11\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %10\n\t"
          "s_mov_b32 m0, %12\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %10\n\t"
          "s_mov_b32 m0, %13\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, %10\n\t"
          "s_mov_b32 m0, %14\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, %10\n\t"
          "s_mov_b32 m0, %15\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %5, %10\n\t"
          "s_mov_b32 m0, %16\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %6, %10\n\t"
          "s_mov_b32 m0, %17\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %7, %10\n\t"
          "s_mov_b32 m0, %18\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %8, %10\n\t"
          "s_mov_b32 m0, %19\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %9, %10\n\t"
          "s_mov_b32 m0, %0"
          : "=&s"(saved)
          : "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "v"(vo[4]), "v"(vo[5]), "v"(vo[6]), "v"(vo[7]),
            "v"((uint32_t)off_b), "s"(kvb), "s"(la[0]), "s"(la[1]), "s"(la[2]), "s"(la[3]), "s"(la[4]),
            "s"(la[5]), "s"(la[6]), "s"(la[7]), "s"(lb));
    } else {
#pragma unroll
      for (int jj = 0; jj < kPerWave; ++jj) issue(jj, tile, kvb, wave);
    }
  }
};

// A wave's copies of one later chunk, issued one at a time between MFMAs
// (issue(jj) does nothing when `more` is false).  Used where registers
// allow it: in the attention kernel the held state made the allocator
// spill the O^T accumulator.
template <int DK, int DV, int NW, bool K64>
struct LaterCopies {
  RowGather<DK, DV, NW, K64> g;
  uint16_t* tile;
  const uint16_t* kvb;
  int wave;
  bool more;
  static constexpr int kPerWave = RowGather<DK, DV, NW, K64>::kPerWave;
  __device__ __forceinline__ void issue(int jj) const {
    if (more) g.issue(jj, tile, kvb, wave);
  }
};

struct NoCopies {
  static constexpr int kPerWave = 0;
  __device__ __forceinline__ void issue(int) const {}
};

template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

template <int DK, int DV, int NW>
struct RowState {
  v16f o[Cfg<DK, DV, NW>::kNT];
  float m_ref;   // softmax reference of this lane's head (log2 units), fixed during a pass
  float m_seen;  // largest logit seen (log2 units)
  float l_sum;   // this half's share of the softmax denominator
};

// S^T = C.Q^T of one chunk (32 gathered rows x this wave's 32 heads): lane
// (half, col) gets head col at rows 8*(j/4) + 4*half + j%4, j = 0..15.
template <int DK, int DV, int NW>
__device__ __forceinline__ v16f qk_chunk(const uint16_t* tb, const v8bf (&qb)[DK / 16]) {
  using C = Cfg<DK, DV, NW>;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, col = lane & 31;
  // ---- A operands prefetched kLookA steps ahead
  // Lane (row col, half) reads logical piece 2*ks + half of its row.  The
  // swizzle only flips the low two bits of the piece index, so every part-A
  // address is one of two per-lane bases plus a compile-time offset.
  const int sw = swz_a(col);
  const uint16_t* a_even = tb + (col * C::kRA + (half ^ sw)) * 8;         // ks even
  const uint16_t* a_odd = tb + (col * C::kRA + ((2 + half) ^ sw)) * 8;    // ks odd
  auto load_a = [&](int ks) {
    if (2 * ks < C::kPA) return *(const v8bf*)((ks & 1 ? a_odd : a_even) + 32 * (ks >> 1));
    return *(const v8bf*)(tb + piece_pos<DK, DV, NW>(col, 2 * ks + half));
  };
  // The S^T chain is written as inline asm so that its accumulator is a
  // VGPR tuple (the compiler would put it in AGPRs, next to O^T, and move an
  // O^T tile out and back every chunk).  The compiler does not see these as
  // MFMAs, so the wait states before the first VALU read of the result are
  // explicit (32x32 XDL result -> VALU read: 18 on gfx950; 21 given).
  v16f st;
  v8bf abuf[kLookA];
#pragma unroll
  for (int j = 0; j < kLookA; ++j) abuf[j] = load_a(j);
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks) {
    const v8bf cur = abuf[ks % kLookA];
    if (ks + kLookA < C::kKS) abuf[ks % kLookA] = load_a(ks + kLookA);
    if (ks == 0)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(st) : "v"(cur), "v"(qb[ks]));
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(st) : "v"(cur), "v"(qb[ks]));
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(st));
  return st;
}

// One chunk of 32 gathered rows: S^T = C.Q^T, softmax weights against the
// fixed reference, O^T += V^T.P^T.  `valid` bit r says row r of the chunk
// holds a selected entry.
template <int DK, int DV, int NW>
__device__ __forceinline__ void attend_chunk(const uint16_t* tb, uint32_t valid, const v8bf (&qb)[DK / 16],
                                             float zscale, RowState<DK, DV, NW>& rs) {
  using C = Cfg<DK, DV, NW>;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const v16f st = qk_chunk<DK, DV, NW>(tb, qb);
  // ---- mask (only a row's last chunk can hold padding), chunk max
  float z[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) z[j] = st[j];
  if (valid != 0xFFFFFFFFu) {   // wave-uniform
    const uint32_t vh = valid >> (4 * half);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 8 * (j >> 2) + (j & 3);       // row minus 4*half
      if (!((vh >> r) & 1u)) z[j] = -INFINITY;
    }
  }
  float mx = z[0];
#pragma unroll
  for (int j = 1; j < 16; ++j) mx = __builtin_fmaxf(mx, z[j]);
  // zscale > 0, so the scaled maximum is the scaled raw maximum
  mx = max_halves(mx) * zscale;
  if (rs.m_ref == -INFINITY) rs.m_ref = mx;
  rs.m_seen = fmaxf(rs.m_seen, mx);
  // ---- probabilities, packed as the P^T operand (K order = S^T row order)
  const float nref = -rs.m_ref;
  v8bf pb[2];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float pj = __builtin_amdgcn_exp2f(__builtin_fmaf(z[j], zscale, nref));
    rs.l_sum += pj;
    pb[j >> 3][j & 7] = (__bf16)pj;
  }
  // ---- O^T += V^T . P^T ; K index k of step kk is row 16*kk + 8*((k%8)/4) + 4*(k/8) + k%4
  // V^T operand of MFMA m (dim tile m/2, K step m%2): lane l needs dim
  // 32t + l%32 at rows 16kk + 4*half + {0..3} (elements 0..3) and
  // 16kk + 8 + 4*half + {0..3} (elements 4..7).  Two transposed reads: lane
  // j of each 16-lane group addresses row (j/4) of the 4-row block at the
  // 4 dims 4*(j%4) of its 16-dim slice.
  // Rows 16kk + 4*half + jl/4 (+8) all share swz_a, so a 64-byte block of
  // 4 pieces stays contiguous; the 4-dim group 4*(jl%4) sits in piece
  // 4t + 2*(g%2) + (jl%4)/2 at element offset 4*(jl%2).
  const int g = lane >> 4, jl = lane & 15;
  const int vrow = 4 * (g >> 1) + (jl >> 2);      // + 16*kk (+ 8 for the high half)
  const int vpiece = 2 * (g & 1) + ((jl & 3) >> 1);
  const int vsub = 4 * (jl & 1);
  // swz_a(16*kk + vrow) does not depend on kk, and the swizzle stays inside
  // the 4-piece group, so addresses are two bases plus compile-time offsets.
  const uint16_t* v_lo = tb + (vrow * C::kRA + (vpiece ^ swz_a(vrow))) * 8 + vsub;
  const uint16_t* v_hi = tb + ((vrow + 8) * C::kRA + (vpiece ^ swz_a(vrow + 8))) * 8 + vsub;
  auto load_v = [&](int m) {
    const int t = m >> 1, kk = m & 1;
    const int off = 16 * kk * C::kRA * 8 + 32 * t;
    const v4bf lo = lds_read_tr16(v_lo + off);
    const v4bf hi = lds_read_tr16(v_hi + off);
    return (v8bf)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  constexpr int kM = 2 * C::kNT;
  v8bf vbuf[kLookV];
#pragma unroll
  for (int j = 0; j < kLookV; ++j) vbuf[j] = load_v(j);
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    const v8bf cur = vbuf[m % kLookV];
    if (m + kLookV < kM) vbuf[m % kLookV] = load_v(m + kLookV);
    rs.o[m >> 1] = mfma_bf16_32x32x16(cur, pb[m & 1], rs.o[m >> 1]);
  }
}

// attend_chunk for the shapes whose rows are gathered one wave instruction
// per row (Dv = 512), with part of the softmax hidden behind the PV MFMAs.
// Counters of attend_chunk: the matrix cores were busy 41% of the kernel and
// co-issued with the VALU in only 1.3% of cycles, since QK, softmax and PV
// ran one after the other.  Here the PV product runs K step 0 (rows 0..15:
// weights 0..7 of each lane) over all 16 dim tiles, then K step 1; the
// weights of K step 1 are computed in the gaps of the first 8 MFMAs of step
// 0.  Each gap's work stays where it is placed (sched_barrier), so the V^T
// operand loads keep their short lookahead.  Every accumulator and the
// softmax sum see the same operations in the same order as in attend_chunk,
// so the results are the same bits.
template <int DK, int DV, int NW>
__device__ __forceinline__ void attend_chunk_ov(const uint16_t* tb, uint32_t valid, const v8bf (&qb)[DK / 16],
                                                float zscale, RowState<DK, DV, NW>& rs) {
  using C = Cfg<DK, DV, NW>;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const v16f st = qk_chunk<DK, DV, NW>(tb, qb);
  float z[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) z[j] = st[j];
  if (valid != 0xFFFFFFFFu) {   // wave-uniform
    const uint32_t vh = valid >> (4 * half);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 8 * (j >> 2) + (j & 3);
      if (!((vh >> r) & 1u)) z[j] = -INFINITY;
    }
  }
  float mx = z[0];
#pragma unroll
  for (int j = 1; j < 16; ++j) mx = __builtin_fmaxf(mx, z[j]);
  mx = max_halves(mx) * zscale;
  if (rs.m_ref == -INFINITY) rs.m_ref = mx;
  rs.m_seen = fmaxf(rs.m_seen, mx);
  const float nref = -rs.m_ref;
  v8bf pb[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float pj = __builtin_amdgcn_exp2f(__builtin_fmaf(z[j], zscale, nref));
    rs.l_sum += pj;
    pb[0][j] = (__bf16)pj;
  }
  const int g = lane >> 4, jl = lane & 15;
  const int vrow = 4 * (g >> 1) + (jl >> 2);
  const int vpiece = 2 * (g & 1) + ((jl & 3) >> 1);
  const int vsub = 4 * (jl & 1);
  const uint16_t* v_lo = tb + (vrow * C::kRA + (vpiece ^ swz_a(vrow))) * 8 + vsub;
  const uint16_t* v_hi = tb + ((vrow + 8) * C::kRA + (vpiece ^ swz_a(vrow + 8))) * 8 + vsub;
  // MFMA n: K step kk = n / kNT over dim tile t = n % kNT
  auto load_v = [&](int n) {
    const int kk = n / C::kNT, t = n % C::kNT;
    const int off = 16 * kk * C::kRA * 8 + 32 * t;
    const v4bf lo = lds_read_tr16(v_lo + off);
    const v4bf hi = lds_read_tr16(v_hi + off);
    return (v8bf)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  constexpr int kM = 2 * C::kNT;
  v8bf vbuf[kLookV];
#pragma unroll
  for (int j = 0; j < kLookV; ++j) vbuf[j] = load_v(j);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int n = 0; n < kM; ++n) {
    const v8bf cur = vbuf[n % kLookV];
    if (n + kLookV < kM) vbuf[n % kLookV] = load_v(n + kLookV);
    const int kk = n / C::kNT, t = n % C::kNT;
    rs.o[t] = mfma_bf16_32x32x16(cur, pb[kk], rs.o[t]);
    if (n < 8) {
      const int j = 8 + n;
      const float pj = __builtin_amdgcn_exp2f(__builtin_fmaf(z[j], zscale, nref));
      rs.l_sum += pj;
      pb[1][j - 8] = (__bf16)pj;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int DK, int DV, int NW, bool kPaged>
__global__ void __launch_bounds__(NW * kWave, 1) sparse_mla_kernel(AttnArgs a) {
  using C = Cfg<DK, DV, NW>;
  // Three LDS tiles as separate objects so the compiler can tell the tile
  // being read from the tiles being filled by DMA.
  __shared__ __attribute__((aligned(16))) uint16_t tile0[C::kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t tile1[C::kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t tile2[C::kTileElems];
  __shared__ int32_t sidx[kMaxSlots];
  __shared__ int redo;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  // Workgroup -> (row b * rows + i, split).  Dispatch places workgroup id
  // on XCD id % 8; the splits of a row read the same Q (147 KB for 128
  // heads) and their partials are combined together, so they go to one
  // XCD: XCD x takes rows 8j + x, a row's splits consecutively.
  int rowid, sp;
  if (a.nsplit == 1) {
    rowid = blockIdx.x;
    sp = 0;
  } else {
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    sp = j % a.nsplit;
    rowid = (j / a.nsplit) * 8 + xcd;
    if (rowid >= a.B * a.rows) return;   // block-uniform, before any barrier
  }
  const int b = rowid / a.rows;
  const int i = rowid % a.rows;
  const int64_t qrow = (int64_t)b * a.qrows_b + i;

  // Slots of this split, in whole chunks.
  const int per_split = ((a.k + a.nsplit - 1) / a.nsplit + kChunk - 1) / kChunk * kChunk;
  const int slot0 = sp * per_split;
  const int nslots = max(0, min(per_split, a.k - slot0));
  const int nchunks = (nslots + kChunk - 1) / kChunk;

  // Slot j holds the cache row of its token (-1 if the entry is padding or
  // outside the sequence): a row of the sequence's cache, or of the pool.
  // A thread's (at most kMaxSlots / kThreads) index loads all go out before
  // the first is used, so the prologue waits for one memory round trip (two
  // with a page table) rather than one per slot a thread covers.
  const int slen = seq_len_of(a.pk, b, a.S);
  {
    constexpr int kPer = kMaxSlots / C::kThreads;
    const int32_t* ip = a.idx + ((int64_t)b * a.idx_rows_b + i) * a.k + slot0;
    int v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = (int)threadIdx.x + u * C::kThreads;
      v[u] = j < nslots ? ip[j] : -1;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      if (v[u] < 0 || v[u] >= slen) v[u] = -1;
      else if (kPaged) v[u] = (int)cache_row(a.pk, b, a.S, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = (int)threadIdx.x + u * C::kThreads;
      if (j < nchunks * kChunk) sidx[j] = v[u];
    }
  }

  __syncthreads();   // the slot indices are published
  // Q^T operand of this wave's 32 heads, kept in registers for the whole row
  // (loaded after the first chunk's copies are issued, below).
  const int h = wave * 32 + col;
  v8bf qb[C::kKS];

  const uint16_t* kvb = kPaged ? a.kv : a.kv + (int64_t)b * a.S * DK;
  RowState<DK, DV, NW> rs;
  rs.m_ref = -INFINITY;
  rs.m_seen = -INFINITY;
  const float zscale = a.sm_scale * kLog2e;
  constexpr int ndma = C::kDma / NW;   // DMA instructions per wave per chunk

  // Chunk c lives in tile c % 3.  DMA for chunk c+2 is issued once every wave
  // has passed the barrier of chunk c (so nobody still reads chunk c-1's
  // tile); before that barrier each wave waits until its own part of chunk c
  // has landed while chunk c+1's DMA stays in flight.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto gather = [&](int c, uint16_t* fill, int ra, int rb) {
    if constexpr (C::kRowDma) {
      RowGather<DK, DV, NW, kPaged> g;
      g.init(ra, rb, wv);
      g.issue_all(fill, kvb, wv);
    } else {
      ChunkGather<DK, DV, NW> g;
      g.init(fill, kvb, ra);
      g.issue_all();
    }
  };
  auto rb_of = [&](int c) {
    if constexpr (C::kRowDma) return sidx[c * kChunk + RowGather<DK, DV, NW, kPaged>::row_b(wv, lane)];
    else return 0;
  };
  auto step = [&](int c, const uint16_t* cur, uint16_t* fill) {
    // The slot indices are read before the barrier (they do not change after
    // the prologue), so their LDS latency overlaps the wait.
    const int cn = min(c + 2, nchunks - 1);
    const int rv = sidx[c * kChunk + (lane & 31)];
    const int ra = sidx[cn * kChunk + (lane & 31)];
    const int rb = rb_of(cn);
    // Each wave waits until its own copies of chunk c landed (chunk c+1's
    // stay in flight); the barrier then publishes the tile.  A compiler-level
    // memory barrier keeps LDS accesses on their side of it; the tile
    // refilled next was last read (and consumed) in chunk c-1.
    if (c + 1 < nchunks) wait_vm<ndma>(); else wait_vm<0>();
    asm volatile("s_barrier" ::: "memory");
    const uint32_t valid = (uint32_t)__builtin_amdgcn_ballot_w64(lane < kChunk && rv >= 0);
    if constexpr (C::kRowDma) {
      // Waves 0-1 issue their copies of chunk c+2 before attending chunk c,
      // waves 2-3 after it, so that 18 rather than 36 copy instructions
      // reach the CU's memory pipeline at once (0.5-1% faster prefill; the
      // per-wave issue order, and so every wait count, is unchanged).
      if (c + 2 < nchunks && wv < 2) gather(c + 2, fill, ra, rb);
      if (valid != 0u) attend_chunk_ov<DK, DV, NW>(cur, valid, qb, zscale, rs);
      if (c + 2 < nchunks && wv >= 2) gather(c + 2, fill, ra, rb);
    } else {
      if (c + 2 < nchunks) gather(c + 2, fill, ra, rb);
      if (valid != 0u) attend_chunk<DK, DV, NW>(cur, valid, qb, zscale, rs);
    }
  };

  // The first chunk's copies go out before the Q^T loads, so that the
  // 147 KB of Q^T (128 heads) and the first rows arrive together.  The empty
  // asm uses below make the compiler wait for Q^T right here (its wait also
  // covers chunk 0's copies, issued earlier), before chunk 1's copies and
  // the loop: the compiler cannot see the copies, and a Q^T wait left to it
  // inside the loop would wait for every copy in flight.
  if (nchunks > 0) gather(0, tile0, sidx[lane & 31], rb_of(0));
  {
    const uint16_t* qp = a.q + (qrow * a.H + min(h, a.H - 1)) * DK + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::kKS; ++ks) {
      v8bf v = *(const v8bf*)(qp + 16 * ks);
      if (h >= a.H) v = (v8bf){};
      qb[ks] = v;
    }
  }
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks) asm volatile("" ::"v"(qb[ks]));
  if (nchunks > 1) gather(1, tile1, sidx[kChunk + (lane & 31)], rb_of(1));

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int t = 0; t < C::kNT; ++t) rs.o[t] = (v16f){};
    rs.l_sum = 0.f;
    if (pass > 0) {
      if (nchunks > 0) gather(0, tile0, sidx[lane & 31], rb_of(0));
      if (nchunks > 1) gather(1, tile1, sidx[kChunk + (lane & 31)], rb_of(1));
    }
    for (int c = 0; c < nchunks; c += 3) {
      step(c, tile0, tile2);
      if (c + 1 >= nchunks) break;
      step(c + 1, tile1, tile0);
      if (c + 2 >= nchunks) break;
      step(c + 2, tile2, tile1);
    }
    // A logit far above its head's reference: redo the row with the true max.
    wait_dma();
    if (threadIdx.x == 0) redo = 0;
    __syncthreads();
    if (rs.m_seen > rs.m_ref + kRefHeadroom) redo = 1;
    __syncthreads();
    if (!redo) break;
    rs.m_ref = rs.m_seen;
  }

  // ---- epilogue
  const float l_tot = sum_halves(rs.l_sum);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (rs.m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
  // The row's output, or with splits this split's normalised output in bf16
  // (the merge weights sum to 1, so this adds at most one more bf16 rounding
  // to the result; it halves the partial traffic of the decode step).  Both
  // are [H][Dv] blocks, so a wave's 32 heads are 32 KB of contiguous memory.
  uint16_t* const ob = a.nsplit == 1 ? a.out + qrow * a.H * DV
                                     : a.part_o + ((int64_t)rowid * a.nsplit + sp) * a.H * DV;
  if constexpr (C::kRowDma) {
    // Staged through LDS (the ring tiles are free once the row is done:
    // every copy has landed and the redo check's barriers have passed), so
    // that each store instruction writes two whole 512-byte head-row halves
    // rather than 16 bytes of each of 32 rows.  Wave w uses a 16.5 KB
    // region of tile0 (w < 2) or tile1; rows are padded to 264 elements
    // (132 dwords) so the 8-byte writes of the 32 heads spread over the
    // banks.  Half p of the dims goes per pass.
    constexpr int kHalf = DV / 2, kStride = kHalf + 8;
    static_assert(2 * 32 * kStride <= C::kTileElems, "two waves' staging fits one tile");
    uint16_t* stg = (wave < 2 ? tile0 : tile1) + (wave & 1) * 32 * kStride;
    const int h0 = wave * 32;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
      for (int t = p * C::kNT / 2; t < (p + 1) * C::kNT / 2; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * t + 8 * g + 4 * half - p * kHalf;
          uint2 pk;
          pk.x = pack_bf16x2(rs.o[t][4 * g + 0] * inv, rs.o[t][4 * g + 1] * inv);
          pk.y = pack_bf16x2(rs.o[t][4 * g + 2] * inv, rs.o[t][4 * g + 3] * inv);
          *(uint2*)(stg + col * kStride + d) = pk;
        }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int hh = 2 * i + half;
        const uint4 v = *(const uint4*)(stg + hh * kStride + 8 * col);
        if (h0 + hh < a.H) *(uint4*)(ob + (int64_t)(h0 + hh) * DV + p * kHalf + 8 * col) = v;
      }
    }
  } else if (h < a.H) {
    uint16_t* op = ob + (int64_t)h * DV;
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
  }
  if (h < a.H && half == 0) {
    if (a.nsplit == 1) {
      if (a.lse) a.lse[qrow * a.H + h] = lse_v;
    } else {
      a.part_lse[((int64_t)rowid * a.nsplit + sp) * a.H + h] = lse_v;
    }
  }
}

// Forward indexer KL on the selected set (page "6.2 DSA Continued
// Pre-Training: Warm-up and Sparse Stages", sparse stage; the analysis page,
// Sec. 1.1 Eq. (4)).  For query row t with selection S:
//   P_s  = sum_h exp(z_hs - lse_h)     (attention weights of all heads, z_hs =
//                                       sm_scale q_h . c_s, lse_h the attention's)
//   p_s  = P_s / T, T = sum_s P_s      (L1 normalisation along the sequence)
//   ln q_s = I_s - LSE_I,  LSE_I = log sum_{s in S} exp(I_s)
//   KL   = sum_s p_s (ln p_s - ln q_s) = A / T - ln T,
//          A = sum_s P_s (ln P_s - I_s + LSE_I).
// One workgroup per row: the selected rows are gathered through the same
// three-tile DMA ring as the attention.  The logits are computed as
// S = Q.C^T (the attention's operands swapped, heads on M, keys on N), so
// lane (half, col) holds 16 heads of key col and the head sum is lane-local
// plus one half swap.  The four waves' sums meet in a two-chunk LDS ring
// that each wave folds (8 keys each) one chunk later; the tile barrier
// orders the accesses.
// `cp.issue(jj)` issues this wave's copy instruction jj (of CP::kPerWave)
// for a later chunk, spread evenly over the K steps so that the memory
// pipeline drains the copies while the matrix core works.
template <int DK, int DV, int NW, typename CP>
__device__ __forceinline__ v16f qk_chunk_heads(const uint16_t* tb, const v8bf (&qb)[DK / 16], const CP& cp) {
  using C = Cfg<DK, DV, NW>;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, col = lane & 31;
  const int sw = swz_a(col);
  const uint16_t* a_even = tb + (col * C::kRA + (half ^ sw)) * 8;
  const uint16_t* a_odd = tb + (col * C::kRA + ((2 + half) ^ sw)) * 8;
  auto load_b = [&](int ks) {
    if (2 * ks < C::kPA) return *(const v8bf*)((ks & 1 ? a_odd : a_even) + 32 * (ks >> 1));
    return *(const v8bf*)(tb + piece_pos<DK, DV, NW>(col, 2 * ks + half));
  };
  v16f st;
  v8bf bbuf[kLookA];
#pragma unroll
  for (int j = 0; j < kLookA; ++j) bbuf[j] = load_b(j);
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks) {
    const v8bf cur = bbuf[ks % kLookA];
    if (ks + kLookA < C::kKS) bbuf[ks % kLookA] = load_b(ks + kLookA);
    if (ks == 0)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(st) : "v"(qb[ks]), "v"(cur));
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(st) : "v"(qb[ks]), "v"(cur));
    if constexpr (CP::kPerWave > 0) {
#pragma unroll
      for (int jj = 0; jj < CP::kPerWave; ++jj)
        if (jj * C::kKS / CP::kPerWave == ks) cp.issue(jj);
    }
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(st));
  return st;
}

template <int DK, int DV, int NW, bool kPaged>
__global__ void __launch_bounds__(NW * kWave, 1) indexer_kl_kernel(KlArgs ka) {
  using C = Cfg<DK, DV, NW>;
  const AttnArgs& a = ka.at;
  __shared__ __attribute__((aligned(16))) uint16_t tile0[C::kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t tile1[C::kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t tile2[C::kTileElems];
  __shared__ int32_t sidx[kMaxSlots];
  __shared__ float isc[kMaxSlots];
  __shared__ float ksum[2][NW][kChunk];
  __shared__ float red[2][NW];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int rowid = blockIdx.x;
  const int b = rowid / a.rows;
  const int i = rowid % a.rows;
  const int64_t qrow = (int64_t)b * a.qrows_b + i;
  const int nchunks = (a.k + kChunk - 1) / kChunk;

  // slots: cache rows (or -1) and the index scores of their tokens
  const int slen = seq_len_of(a.pk, b, a.S);
  const float* srow = ka.scores + ((int64_t)b * ka.sc_rows_b + i) * ka.ld;
  {
    // all of a thread's index loads first, then all of its score loads
    constexpr int kPer = kMaxSlots / C::kThreads;
    const int32_t* ip = a.idx + ((int64_t)b * a.idx_rows_b + i) * a.k;
    int t[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = (int)threadIdx.x + u * C::kThreads;
      t[u] = j < a.k ? ip[j] : -1;
    }
    int v[kPer];
    float iv[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const bool ok = t[u] >= 0 && t[u] < slen;
      iv[u] = ok ? srow[t[u]] : -INFINITY;
      v[u] = !ok ? -1 : kPaged ? (int)cache_row(a.pk, b, a.S, t[u]) : t[u];
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = (int)threadIdx.x + u * C::kThreads;
      if (j < nchunks * kChunk) {
        sidx[j] = v[u];
        isc[j] = iv[u];
      }
    }
  }
  __syncthreads();
  // LSE_I over the selected set: block max, then block sum (fixed orders)
  float mI = -INFINITY;
  for (int j = threadIdx.x; j < nchunks * kChunk; j += C::kThreads) mI = fmaxf(mI, isc[j]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) mI = fmaxf(mI, __shfl_xor(mI, d, kWave));
  if (lane == 0) red[0][wave] = mI;
  __syncthreads();
  mI = red[0][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) mI = fmaxf(mI, red[0][w]);
  float sI = 0.f;
  if (mI > -INFINITY)
    for (int j = threadIdx.x; j < nchunks * kChunk; j += C::kThreads)
      if (isc[j] > -INFINITY) sI += __expf(isc[j] - mI);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) sI += __shfl_xor(sI, d, kWave);
  if (lane == 0) red[1][wave] = sI;
  __syncthreads();
  sI = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) sI += red[1][w];
  const float lse_i = mI + __logf(sI);
  if (!(mI > -INFINITY)) {   // empty selection (block-uniform)
    if (threadIdx.x == 0) ka.kl[qrow] = 0.f;
    return;
  }

  // Q of this wave's 32 heads (A operand: lane holds head 32*wave + col), and
  // the log-sum-exp (log2 units) of the 16 heads of this lane's result rows
  // 32*wave + 8*(j/4) + 4*half + j%4; heads past H weigh 0.
  const int h = wave * 32 + col;
  v8bf qb[C::kKS];
  {
    const uint16_t* qp = a.q + (qrow * a.H + min(h, a.H - 1)) * DK + 8 * half;
#pragma unroll
    for (int ks = 0; ks < C::kKS; ++ks) {
      v8bf v = *(const v8bf*)(qp + 16 * ks);
      if (h >= a.H) v = (v8bf){};
      qb[ks] = v;
    }
  }
  float lse2[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int hj = wave * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
    lse2[j] = hj < a.H ? a.lse[qrow * a.H + hj] * kLog2e : INFINITY;   // +inf: weight 0
  }
  const float zscale = a.sm_scale * kLog2e;
  wait_vm<0>();
  __syncthreads();

  const uint16_t* kvb = kPaged ? a.kv : a.kv + (int64_t)b * a.S * DK;
  constexpr int ndma = C::kDma / NW;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto gather = [&](uint16_t* fill, int ra, int rb) {
    if constexpr (C::kRowDma) {
      RowGather<DK, DV, NW, kPaged> g;
      g.init(ra, rb, wv);
      g.issue_all(fill, kvb, wv);
    } else {
      ChunkGather<DK, DV, NW> g;
      g.init(fill, kvb, ra);
      g.issue_all();
    }
  };
  auto rb_of = [&](int c) {
    if constexpr (C::kRowDma) return sidx[c * kChunk + RowGather<DK, DV, NW, kPaged>::row_b(wv, lane)];
    else return 0;
  };
  // Each wave folds kChunk / NW keys of a chunk (lanes below that count).
  constexpr int kFold = kChunk / NW;
  float acc_a = 0.f, acc_t = 0.f;   // this lane's share of A and T
  auto fold = [&](int c) {
    if (lane < kFold) {
      const int r = wave * kFold + lane;
      float ps = ksum[c & 1][0][r];
#pragma unroll
      for (int w = 1; w < NW; ++w) ps += ksum[c & 1][w][r];
      const int slot = c * kChunk + r;
      if (sidx[slot] >= 0 && ps > 0.f) {
        acc_a += ps * (__logf(ps) - isc[slot] + lse_i);
        acc_t += ps;
      }
    }
  };
  auto step = [&](int c, const uint16_t* cur, uint16_t* fill) {
    const int cn = min(c + 2, nchunks - 1);
    const int rv = sidx[c * kChunk + (lane & 31)];
    const int ra = sidx[cn * kChunk + (lane & 31)];
    const int rb = rb_of(cn);
    if (c + 1 < nchunks) wait_vm<ndma>(); else wait_vm<0>();
    // the LDS head sums of chunk c-1 must have landed before wave 0 reads them
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    v16f st;
    if constexpr (C::kRowDma) {
      // chunk c+2's copies ride along this chunk's QK steps
      LaterCopies<DK, DV, NW, kPaged> cp;
      cp.g.init(ra, rb, wv);
      cp.tile = fill;
      cp.kvb = kvb;
      cp.wave = wv;
      cp.more = c + 2 < nchunks;
      if (c > 0) fold(c - 1);
      st = qk_chunk_heads<DK, DV, NW>(cur, qb, cp);
    } else {
      if (c + 2 < nchunks) gather(fill, ra, rb);
      if (c > 0) fold(c - 1);
      st = qk_chunk_heads<DK, DV, NW>(cur, qb, NoCopies{});
    }
    const bool kval = rv >= 0;   // this lane's key (col) is a selected entry
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) ps += __builtin_amdgcn_exp2f(__builtin_fmaf(st[j], zscale, -lse2[j]));
    ps = sum_halves(ps);   // the wave's 32 heads
    if (lane < kChunk) ksum[c & 1][wave][lane] = kval ? ps : 0.f;
  };

  if (nchunks > 0) gather(tile0, sidx[lane & 31], rb_of(0));
  if (nchunks > 1) gather(tile1, sidx[kChunk + (lane & 31)], rb_of(1));
  for (int c = 0; c < nchunks; c += 3) {
    step(c, tile0, tile2);
    if (c + 1 >= nchunks) break;
    step(c + 1, tile1, tile0);
    if (c + 2 >= nchunks) break;
    step(c + 2, tile2, tile1);
  }
  wait_dma();
  __syncthreads();
  fold(nchunks - 1);
  // lanes past kFold hold zeros; fixed butterflies and a fixed wave order
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    acc_a += __shfl_xor(acc_a, d, kWave);
    acc_t += __shfl_xor(acc_t, d, kWave);
  }
  if (lane == 0) {
    red[0][wave] = acc_a;
    red[1][wave] = acc_t;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float ta = red[0][0], tt = red[1][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      ta += red[0][w];
      tt += red[1][w];
    }
    ka.kl[qrow] = tt > 0.f ? ta / tt - __logf(tt) : 0.f;
  }
}

// Merge split partials: lse = log sum_j exp(lse_j), o = sum_j exp(lse_j - lse) o_j.
template <int DV>
__global__ void __launch_bounds__(DV / 8) mla_combine_kernel(AttnArgs a) {
  // (row, head) on the XCD that ran the row's splits (rows 8j + x on XCD x)
  const int xcd = blockIdx.x & 7, jw = blockIdx.x >> 3;
  const int rowid = (jw / a.H) * 8 + xcd;
  const int h = jw % a.H;
  if (rowid >= a.B * a.rows) return;
  const int b = rowid / a.rows, i = rowid % a.rows;
  const int64_t qrow = (int64_t)b * a.qrows_b + i;
  const float* pl = a.part_lse + (int64_t)rowid * a.nsplit * a.H + h;
  const int d = threadIdx.x * 8;
  const uint16_t* po = a.part_o + ((int64_t)rowid * a.nsplit * a.H + h) * DV + d;
  const int64_t pstride = (int64_t)a.H * DV;
  // One wave per (row, head), 8 dims per lane in 16-byte loads.  Every
  // split's log-sum-exp and partial are loaded before the first is used, so
  // a lane waits for one memory round trip, not one per split (an empty
  // split's partial is zeros, written by the split kernel).
  float lv[kMaxSplits];
  uint4 pv[kMaxSplits];
#pragma unroll
  for (int j = 0; j < kMaxSplits; ++j)
    if (j < a.nsplit) {
      lv[j] = pl[(int64_t)j * a.H];
      pv[j] = *(const uint4*)(po + j * pstride);
    }
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < kMaxSplits; ++j)
    if (j < a.nsplit) mx = fmaxf(mx, lv[j]);
  float den = 0.f;
  if (mx > -INFINITY) {
#pragma unroll
    for (int j = 0; j < kMaxSplits; ++j)
      if (j < a.nsplit) den += __expf(lv[j] - mx);
  }
  const float lse = mx > -INFINITY ? mx + __logf(den) : -INFINITY;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (mx > -INFINITY) {
#pragma unroll
    for (int j = 0; j < kMaxSplits; ++j) {
      if (j >= a.nsplit || lv[j] == -INFINITY) continue;
      const float wj = __expf(lv[j] - lse);
      const uint32_t w4[4] = {pv[j].x, pv[j].y, pv[j].z, pv[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += wj * __uint_as_float(w4[e] << 16);
        acc[2 * e + 1] += wj * __uint_as_float(w4[e] & 0xFFFF0000u);
      }
    }
  }
  uint4 pk;
  pk.x = pack_bf16x2(acc[0], acc[1]);
  pk.y = pack_bf16x2(acc[2], acc[3]);
  pk.z = pack_bf16x2(acc[4], acc[5]);
  pk.w = pack_bf16x2(acc[6], acc[7]);
  *(uint4*)(a.out + (qrow * a.H + h) * DV + d) = pk;
  if (a.lse && threadIdx.x == 0) a.lse[qrow * a.H + h] = lse;
}

template <int DK, int DV, int NW>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t st) {
  const int nrow = a.B * a.rows, nrow8 = (nrow + 7) / 8;
  const unsigned grid = a.nsplit == 1 ? (unsigned)nrow : (unsigned)(8 * nrow8 * a.nsplit);
  if (a.pk.page_table)
    hipLaunchKernelGGL((sparse_mla_kernel<DK, DV, NW, true>), dim3(grid), dim3(NW * kWave), 0, st, a);
  else
    hipLaunchKernelGGL((sparse_mla_kernel<DK, DV, NW, false>), dim3(grid), dim3(NW * kWave), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL((mla_combine_kernel<DV>), dim3((unsigned)(8 * nrow8 * a.H)), dim3(DV / 8), 0, st, a);
  return hipGetLastError();
}

}  // namespace

bool attn_dims_supported(int H, int Dk, int Dv) {
  if (Dk == 576 && Dv == 512) return H >= 1 && H <= 128;
  if (Dk == 80 && Dv == 64) return H >= 1 && H <= 32;
  return false;
}

template <int DK, int DV, int NW>
hipError_t launch_kl_cfg(const KlArgs& ka, hipStream_t st) {
  const unsigned grid = (unsigned)(ka.at.B * ka.at.rows);
  if (ka.at.pk.page_table)
    hipLaunchKernelGGL((indexer_kl_kernel<DK, DV, NW, true>), dim3(grid), dim3(NW * kWave), 0, st, ka);
  else
    hipLaunchKernelGGL((indexer_kl_kernel<DK, DV, NW, false>), dim3(grid), dim3(NW * kWave), 0, st, ka);
  return hipGetLastError();
}

hipError_t launch_sparse_mla(const AttnArgs& a, hipStream_t st) {
  if (a.rows <= 0 || a.B <= 0) return hipSuccess;
  if (a.Dk == 576 && a.Dv == 512) return launch_cfg<576, 512, 4>(a, st);
  if (a.Dk == 80 && a.Dv == 64) return launch_cfg<80, 64, 1>(a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_indexer_kl(const KlArgs& ka, hipStream_t st) {
  if (ka.at.rows <= 0 || ka.at.B <= 0) return hipSuccess;
  if (ka.at.Dk == 576 && ka.at.Dv == 512) return launch_kl_cfg<576, 512, 4>(ka, st);
  if (ka.at.Dk == 80 && ka.at.Dv == 64) return launch_kl_cfg<80, 64, 1>(ka, st);
  return hipErrorInvalidValue;
}

}  // namespace dsa
