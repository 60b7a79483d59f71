// Device-side helpers shared by the DSA kernels (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// 16x16x128 FP8(E4M3) x FP8(E4M3) -> fp32 MFMA with unit block scales
// (E8M0 127 = 2^0).  Operand layout (verified on gfx950): lane l holds row
// (A) / column (B) l%16 and K bytes [32*(l/16), 32*(l/16)+32); the result
// lane l holds rows 4*(l/16)+r, r=0..3, of column l%16.
__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 127, 0, 127);
}

// The same MFMA with E8M0 block scales for A (bits 7..0 of sa, value
// 2^(sa - 127)).  Measured on gfx950: the scale held by lane 16*sb + rho
// multiplies, in A row rho, bytes [16*(sb/2), 16*(sb/2) + 16) of the lanes
// 16*(2*(sb%2)) + rho and 16*(2*(sb%2) + 1) + rho.  In terms of the byte
// index k = 32*(l/16) + j of the layout above, block sb is the set of k
// with 2*((k%32)/16) + k/64 == sb.
__device__ __forceinline__ v4f mfma_fp8_16x16x128_sa(const v8i& a, int sa, const v8i& b) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, sa, 0, 127);
}

// 32x32x16 bf16 MFMA.  Lane l holds row (A) / column (B) l%32 and K elements
// [8*(l/32), 8*(l/32)+8); the result element j of lane l is row
// 8*(j/4) + 4*(l/32) + j%4 of column l%32.
__device__ __forceinline__ v16f mfma_bf16_32x32x16(const v8bf& a, const v8bf& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Exchange across wave halves.  For lanes l < 32 the result is
// x[l] + x[l+32]; for lanes l >= 32 it is y[l-32] + y[l].
__device__ __forceinline__ float reduce_halves(float x, float y) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Same across 16-lane rows: lanes in rows 0 and 2 get x[l] + x[l+16];
// lanes in rows 1 and 3 get y[l-16] + y[l].
__device__ __forceinline__ float reduce_rows16(float x, float y) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reduce-scatter of four per-lane partials over the four 16-lane rows of a
// wave: afterwards lane l (row g = l/16, column n = l%16) holds
// sum_{g'} p[g][g'*16 + n].  The addition tree is fixed, so every caller
// gets bit-identical sums for the same partials.
__device__ __forceinline__ float reduce_scatter4(float p0, float p1, float p2, float p3) {
  const float a = reduce_halves(p0, p2);   // rows 0,1: p0 sums; rows 2,3: p2 sums
  const float b = reduce_halves(p1, p3);   // rows 0,1: p1 sums; rows 2,3: p3 sums
  return reduce_rows16(a, b);              // row 0:p0 row 1:p1 row 2:p2 row 3:p3
}

// ds_read_b64_tr_b16 (verified on gfx950): within each 16-lane group, lane
// c returns element c%4 of the 8-byte chunks addressed by lanes c/4, c/4+4,
// c/4+8 and c/4+12 of the group.  If lanes 4i..4i+3 address 4 consecutive
// columns each of row i of a 4 x 16 bf16 block, lane c receives column c.
__device__ __forceinline__ v4bf lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) v4bf*)(p));
}

__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float max_rows16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS DMA (global_load_lds) issued from inline asm: each lane copies 16
// (or 4) bytes from `src` to lds_base + 16*lane (4*lane); lds_base must be
// wave-uniform.  The compiler's wait insertion cannot tell separate LDS
// buffers apart: it would make every LDS read wait for all DMA in flight,
// including prefetches into other buffers.  Copies issued here are invisible
// to it, so the kernels await completion explicitly (wait_dma / a counted
// s_waitcnt vmcnt) before the barrier that publishes a buffer.  M0 is saved
// and restored around the copy.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}
__device__ __forceinline__ void dma_x4(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(lds_base) : "memory");
}
__device__ __forceinline__ void dma_x1(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(lds_base) : "memory");
}
// Same copy with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset (the "saddr" form): one VGPR of address per lane.  No memory
// clobber: the caller guarantees that nothing reads or writes the target
// buffer between this copy and the barrier that publishes it (volatile asm
// statements keep their order, so the copy stays between its barriers).
__device__ __forceinline__ void dma_x4_s(uint32_t voff, const void* sbase, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(voff), "s"(sbase), "s"(lds_base));
}
__device__ __forceinline__ void dma_x1_s(uint32_t voff, const void* sbase, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(voff), "s"(sbase), "s"(lds_base));
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace dsa
