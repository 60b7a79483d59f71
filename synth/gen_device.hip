// Seeded synthetic inputs, device side.
//
// Fills device buffers with the same values the host generator (gen.py)
// produces, bit for bit, so that large inputs (hundreds of millions of
// elements) are made in HBM directly while the CPU reference regenerates any
// slice it needs on the host.  Nothing here belongs to the attention method:
// it is a counter-based random source (SplitMix64's output function over a
// Weyl sequence, as published by Steele, Lea & Flood, OOPSLA 2014), an
// Irwin-Hall(12) sum of 20-bit uniforms, and rounding to bf16 / OCP FP8 E4M3.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__host__ __device__ __forceinline__ uint64_t mix64_hd(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Irwin-Hall(12) sample for flat element e of the stream `base`; exact in fp32.
__device__ __forceinline__ float normal_at(uint64_t base, uint64_t e) {
  uint32_t acc = 0;
  const uint64_t e6 = e * 6ull;
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const uint64_t x = mix64(base + (e6 + (uint64_t)(j + 1)) * kGamma);
    acc += (uint32_t)(x & 0xFFFFFull) + (uint32_t)((x >> 32) & 0xFFFFFull);
  }
  const int32_t z = (int32_t)acc - (int32_t)(6 << 20);
  return (float)z * 0x1p-20f;
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// float -> OCP E4M3FN, round to nearest even, saturating at +-448.
__device__ __forceinline__ uint8_t e4m3_rne_sat(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x3C800000u) {                       // |x| >= 2^-6: normal e4m3
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;  // fp32 exp<<3 | 3-bit mantissa
    code = r - (120u << 3);                      // rebias 127 -> 7
    code = code > 0x7Eu ? 0x7Eu : code;          // saturate to 448
  } else {                                        // subnormal: multiples of 2^-9
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  return (uint8_t)(code | sign);
}

__global__ void fill_bf16_kernel(uint64_t base, int64_t start, int64_t n, float mul, uint16_t* out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = bf16_rne(normal_at(base, (uint64_t)(start + i)) * mul);
}

__global__ void fill_f32_kernel(uint64_t base, int64_t start, int64_t n, float mul, float* out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = normal_at(base, (uint64_t)(start + i)) * mul;
}

// One block per token.  scale = amax/448 (1 if amax == 0), code = e4m3(z/scale).
constexpr int kQBlock = 256;
__global__ void __launch_bounds__(kQBlock) quant_tokens_kernel(uint64_t base, int64_t tok0, int tok_len,
                                                                uint8_t* codes, float* scales) {
  __shared__ float red[kQBlock / 64];
  const int64_t tok = tok0 + blockIdx.x;
  const int64_t e0 = tok * (int64_t)tok_len;
  float amax = 0.f;
  for (int j = threadIdx.x; j < tok_len; j += kQBlock)
    amax = fmaxf(amax, fabsf(normal_at(base, (uint64_t)(e0 + j))));
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = red[0];
  for (int w = 1; w < kQBlock / 64; ++w) amax = fmaxf(amax, red[w]);
  const float scale = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  uint8_t* dst = codes + (int64_t)blockIdx.x * tok_len;
  for (int j = threadIdx.x; j < tok_len; j += kQBlock)
    dst[j] = e4m3_rne_sat(__fdiv_rn(normal_at(base, (uint64_t)(e0 + j)), scale));
  if (threadIdx.x == 0) scales[blockIdx.x] = scale;
}

int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  return (int)(g > 65536 ? 65536 : (g < 1 ? 1 : g));
}

}  // namespace

extern "C" {

uint64_t synth_stream_key(uint64_t seed, int32_t tid) { return mix64_hd(seed * kGamma + (uint64_t)tid); }

// out[i] = bf16(z(start+i) * 2^exp2), i < n.  Returns a hipError_t value.
int synth_fill_bf16(uint64_t seed, int32_t tid, int64_t start, int64_t n, int32_t exp2, void* out, void* stream) {
  if (n <= 0) return 0;
  const float mul = ldexpf(1.0f, exp2);
  hipLaunchKernelGGL(fill_bf16_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                     synth_stream_key(seed, tid), start, n, mul, (uint16_t*)out);
  return (int)hipGetLastError();
}

int synth_fill_f32(uint64_t seed, int32_t tid, int64_t start, int64_t n, int32_t exp2, void* out, void* stream) {
  if (n <= 0) return 0;
  const float mul = ldexpf(1.0f, exp2);
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                     synth_stream_key(seed, tid), start, n, mul, (float*)out);
  return (int)hipGetLastError();
}

// Tokens [tok0, tok0+n_tok) of length tok_len; codes [n_tok, tok_len], scales [n_tok].
int synth_fill_e4m3_tokens(uint64_t seed, int32_t tid, int64_t tok0, int64_t n_tok, int32_t tok_len,
                           void* codes, void* scales, void* stream) {
  if (n_tok <= 0) return 0;
  int64_t done = 0;
  while (done < n_tok) {  // grid.x is limited to 2^31-1; chunk anyway to keep launches modest
    const int64_t cnt = (n_tok - done) > (1 << 20) ? (1 << 20) : (n_tok - done);
    hipLaunchKernelGGL(quant_tokens_kernel, dim3((unsigned)cnt), dim3(kQBlock), 0, (hipStream_t)stream,
                       synth_stream_key(seed, tid), tok0 + done, tok_len,
                       (uint8_t*)codes + done * (int64_t)tok_len, (float*)scales + done);
    done += cnt;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

}  // extern "C"
