// FP8 (OCP E4M3, the "FN" variant: bias 7, subnormals, no infinities, 448
// the largest value) expert weights with one fp32 scale per output channel:
// per row of an [out, in] matrix, scale = amax / 448 (1 for an all-zero
// row) and code = E4M3(w / scale), each step in fp32, the division
// correctly rounded, the encoding round-to-nearest-even with saturation at
// 448.  Done once when the weights are loaded.  One wave per row.
#include "moe_internal.h"

namespace moe {

// E4M3 code of an fp32 value: round-to-nearest-even on the 3-bit mantissa
// (subnormals: on multiples of 2^-9), magnitudes that round past 448
// saturate to 448; the sign bit is kept (also for -0).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t abits = bits & 0x7fffffffu;
  const float a = __uint_as_float(abits);
  if (!(a < 448.0f)) return sign | 0x7eu;
  if (a < 0.015625f) {  // below 2^-6: subnormal steps of 2^-9 (the product by 512 is exact)
    const uint32_t m = (uint32_t)rintf(a * 512.0f);  // 0 .. 8; 8 is the smallest normal, code 0x08
    return sign | m;
  }
  // keep 3 mantissa bits, ties to even; a carry moves to the next binade
  const uint32_t r = (abits + 0x7ffffu + ((abits >> 20) & 1u)) & ~0xfffffu;
  const int e = (int)(r >> 23) - 127 + 7;
  const uint32_t m = (r >> 20) & 7u;
  if (e > 15 || (e == 15 && m == 7)) return sign | 0x7eu;  // rounded past 448
  return sign | ((uint32_t)e << 3) | m;
}

template <bool BF16>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const void* __restrict__ w, long rows, int C,
                                                           uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const long base = row * C;
  auto at = [&](int c) -> float {
    return BF16 ? bf16_to_f32(((const uint16_t*)w)[base + c]) : ((const float*)w)[base + c];
  };
  float amax = 0.0f;
  for (int c = lane; c < C; c += 64) amax = fmaxf(amax, fabsf(at(c)));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  for (int c = lane; c < C; c += 64) codes[base + c] = (uint8_t)e4m3_encode(at(c) / s);
  if (lane == 0) scales[row] = s;
}

hipError_t launch_quantize_fp8(const void* w, int bf16, long rows, int C, uint8_t* codes, float* scales,
                               hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const long grid = (rows + 3) / 4;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL(quantize_fp8_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, w, rows, C, codes, scales);
  else
    hipLaunchKernelGGL(quantize_fp8_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, w, rows, C, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
