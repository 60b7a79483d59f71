// Per-token FP8 (OCP E4M3FN) quantisation and the decode cache append (the
// step that feeds the FP8 lightning indexer of the page "DeepSeek-V3.2:
// sparse attention, scaled RL and synthetic agent environments", Sec. 1.1).
//
// Per token: scale = amax / 448 (1 for an all-zero token), then every value
// is divided by the scale (correctly rounded fp32) and rounded to the
// nearest E4M3 value, ties to even, saturating at +-448.  The conversion is
// done in integer arithmetic on the fp32 bit pattern, so it does not depend
// on hardware conversion modes:
//   |y| >= 448          -> 0x7E (saturate)
//   2^-6 <= |y| < 448   -> round the fp32 mantissa to 3 bits at bit 20 (RNE);
//                          code = (exponent - 120) << 3 | mantissa
//   |y| < 2^-6          -> code = rint(|y| * 2^9) in 0..8 (subnormals; 8 is
//                          the smallest normal, 2^-6)
// and the sign bit of y goes to bit 7.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

__device__ __forceinline__ uint32_t e4m3_rne_sat(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {          // >= 448
    code = 0x7Eu;
  } else if (a >= 0x3C800000u) {   // >= 2^-6
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = min((r >> 20) - (120u << 3), 0x7Eu);
  } else {
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  return sign | code;
}

// Four consecutive values of a token as fp32.
template <int DT>
__device__ __forceinline__ float4 load4(const void* base, int64_t elem) {
  if constexpr (DT == 0) {
    return *(const float4*)((const float*)base + elem);
  } else {
    const uint2 w = *(const uint2*)((const uint16_t*)base + elem);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                       __uint_as_float(w.y & 0xFFFF0000u));
  }
}

__device__ __forceinline__ float amax4(const float4& v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

__device__ __forceinline__ uint32_t pack_codes(const float4& v, float scale) {
  return e4m3_rne_sat(__fdiv_rn(v.x, scale)) | (e4m3_rne_sat(__fdiv_rn(v.y, scale)) << 8) |
         (e4m3_rne_sat(__fdiv_rn(v.z, scale)) << 16) | (e4m3_rne_sat(__fdiv_rn(v.w, scale)) << 24);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
  return v;
}

constexpr int kQThreads = 256;

// Output row of token `tok`: (tok / group) * out_stride + out_off + tok % group
// (plain quantisation: group = n_tokens, out_off = 0; cache append: group =
// n_q new tokens per sequence, out_stride = n_kv, out_off = q_pos0).
struct QuantArgs {
  const void* x;
  uint8_t* codes;
  float* scales;
  int64_t n_tokens;
  int32_t len;
  int32_t group;
  int64_t out_stride;
  int64_t out_off;
};

__device__ __forceinline__ int64_t out_row(const QuantArgs& a, int64_t tok) {
  return (tok / a.group) * a.out_stride + a.out_off + tok % a.group;
}

// Short tokens: LPT lanes per token (64 / LPT tokens per wave, 4 waves per
// workgroup), each lane holding V groups of 4 values in registers between
// the amax reduction and the conversion, so the token is read once.
template <int DT, int LPT, int V>
__global__ void __launch_bounds__(kQThreads) quant_wave_kernel(QuantArgs a) {
  constexpr int kTPW = kWave / LPT;   // tokens per wave
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPT;
  const int64_t tok = ((int64_t)blockIdx.x * (kQThreads / kWave) + (threadIdx.x >> 6)) * kTPW + lane / LPT;
  const bool live = tok < a.n_tokens;
  const int64_t in0 = min(tok, a.n_tokens - 1) * a.len;
  float4 v[V];
  float m = 0.f;
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const int j = 4 * (sub + u * LPT);
    v[u] = j < a.len ? load4<DT>(a.x, in0 + j) : make_float4(0.f, 0.f, 0.f, 0.f);
    m = fmaxf(m, amax4(v[u]));
  }
#pragma unroll
  for (int d = LPT / 2; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, kWave));
  if (!live) return;
  const float scale = m > 0.f ? __fdiv_rn(m, 448.f) : 1.f;
  const int64_t orow = out_row(a, tok);
  uint32_t* dst = (uint32_t*)(a.codes + orow * a.len);
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const int j = 4 * (sub + u * LPT);
    if (j < a.len) dst[j >> 2] = pack_codes(v[u], scale);
  }
  if (sub == 0) a.scales[orow] = scale;
}

// One workgroup per token (longer tokens, e.g. a query's H_I x d_I values),
// each thread holding V groups of 4 values.
template <int DT, int V>
__global__ void __launch_bounds__(kQThreads) quant_block_kernel(QuantArgs a) {
  __shared__ float red[kQThreads / kWave];
  const int t = threadIdx.x;
  const int64_t tok = blockIdx.x;
  const int64_t in0 = tok * a.len;
  float4 v[V];
  float m = 0.f;
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const int j = 4 * (t + u * kQThreads);
    v[u] = j < a.len ? load4<DT>(a.x, in0 + j) : make_float4(0.f, 0.f, 0.f, 0.f);
    m = fmaxf(m, amax4(v[u]));
  }
  m = wave_max(m);
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float scale = m > 0.f ? __fdiv_rn(m, 448.f) : 1.f;
  const int64_t orow = out_row(a, tok);
  uint32_t* dst = (uint32_t*)(a.codes + orow * a.len);
#pragma unroll
  for (int u = 0; u < V; ++u) {
    const int j = 4 * (t + u * kQThreads);
    if (j < a.len) dst[j >> 2] = pack_codes(v[u], scale);
  }
  if (t == 0) a.scales[orow] = scale;
}
static_assert(kQThreads / kWave == 4, "block reduction assumes 4 waves");

template <int DT>
hipError_t launch_quant_dt(const QuantArgs& a, hipStream_t st) {
  const int64_t n = a.n_tokens;
  auto waves = [&](int tpw) { return dim3((unsigned)((n + 4 * tpw - 1) / (4 * tpw))); };
  const dim3 blk(kQThreads);
  if (a.len <= 128) hipLaunchKernelGGL((quant_wave_kernel<DT, 32, 1>), waves(2), blk, 0, st, a);
  else if (a.len <= 256) hipLaunchKernelGGL((quant_wave_kernel<DT, 64, 1>), waves(1), blk, 0, st, a);
  else if (a.len <= 512) hipLaunchKernelGGL((quant_wave_kernel<DT, 64, 2>), waves(1), blk, 0, st, a);
  else if (a.len <= 1024) hipLaunchKernelGGL((quant_wave_kernel<DT, 64, 4>), waves(1), blk, 0, st, a);
  else if (a.len <= 2048) hipLaunchKernelGGL((quant_block_kernel<DT, 2>), dim3((unsigned)n), blk, 0, st, a);
  else if (a.len <= 4096) hipLaunchKernelGGL((quant_block_kernel<DT, 4>), dim3((unsigned)n), blk, 0, st, a);
  else if (a.len <= 8192) hipLaunchKernelGGL((quant_block_kernel<DT, 8>), dim3((unsigned)n), blk, 0, st, a);
  else hipLaunchKernelGGL((quant_block_kernel<DT, 16>), dim3((unsigned)n), blk, 0, st, a);
  return hipGetLastError();
}

// Latent rows of the new tokens into the cache, 16 bytes per thread.
__global__ void __launch_bounds__(kQThreads) copy_rows_kernel(const uint16_t* src, uint16_t* dst, int64_t n_rows,
                                                              int32_t row_len, int32_t group, int64_t out_stride,
                                                              int64_t out_off) {
  const int per_row = row_len / 8;
  const int64_t id = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
  if (id >= n_rows * per_row) return;
  const int64_t r = id / per_row;
  const int p = (int)(id % per_row);
  const int64_t orow = (r / group) * out_stride + out_off + r % group;
  *(uint4*)(dst + orow * row_len + 8 * p) = *(const uint4*)(src + r * row_len + 8 * p);
}

}  // namespace

hipError_t launch_quantize(const void* x, int dtype, int64_t n_tokens, int32_t len, int32_t group,
                           int64_t out_stride, int64_t out_off, uint8_t* codes, float* scales, hipStream_t st) {
  if (n_tokens <= 0) return hipSuccess;
  const QuantArgs a{x, codes, scales, n_tokens, len, group, out_stride, out_off};
  return dtype == 0 ? launch_quant_dt<0>(a, st) : launch_quant_dt<1>(a, st);
}

hipError_t launch_copy_rows(const uint16_t* src, uint16_t* dst, int64_t n_rows, int32_t row_len, int32_t group,
                            int64_t out_stride, int64_t out_off, hipStream_t st) {
  if (n_rows <= 0) return hipSuccess;
  const int64_t threads = n_rows * (row_len / 8);
  hipLaunchKernelGGL(copy_rows_kernel, dim3((unsigned)((threads + kQThreads - 1) / kQThreads)), dim3(kQThreads), 0, st,
                     src, dst, n_rows, row_len, group, out_stride, out_off);
  return hipGetLastError();
}

}  // namespace dsa
