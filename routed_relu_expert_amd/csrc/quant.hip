// Expert weight quantisation, done once when the weights are loaded.
//
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

// ---------------------------------------------------------------------------
// MXFP4 (OCP Microscaling Formats v1.0): blocks of 32 consecutive elements of
// a row share the E8M0 scale 2^shared, shared = floor(log2 amax) - 2 clamped
// to [-127, 127] (-127 for an all-zero block), and each element becomes the
// E2M1 code of w / 2^shared, nearest with ties to the even code, saturating
// at 6.  One thread per block.
// ---------------------------------------------------------------------------

// E2M1 code of a value: its magnitude code is the count of midpoints below
// it, a tie (a value on a midpoint) going to the even code: 0.25 -> 0, 0.75
// -> 1.0, 1.25 -> 1.0, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4; past 5 the
// largest magnitude 6.  The sign bit is kept (also for -0).
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  const float a = fabsf(v);
  const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return m | ((__float_as_uint(v) >> 28) & 8u);
}

template <bool BF16>
__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(const void* __restrict__ w, int G, int R, int C,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  const int nbr = C / kMxBlock;  // blocks per row
  const long n = (long)G * R * nbr;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const long gr = i / nbr;  // matrix row g * R + r
    const int j = (int)(i - gr * nbr);
    const long g = gr / R;
    const int r = (int)(gr - g * R);
    float v[kMxBlock];
    if (BF16) {
      const uint4* p = (const uint4*)((const uint16_t*)w + gr * C + j * kMxBlock);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 u = p[q];
        const uint32_t h[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[8 * q + 2 * t] = bf16_to_f32(h[t] & 0xffffu);
          v[8 * q + 2 * t + 1] = bf16_to_f32(h[t] >> 16);
        }
      }
    } else {
      const float4* p = (const float4*)((const float*)w + gr * C + j * kMxBlock);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 u = p[q];
        v[4 * q] = u.x;
        v[4 * q + 1] = u.y;
        v[4 * q + 2] = u.z;
        v[4 * q + 3] = u.w;
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < kMxBlock; ++q) amax = fmaxf(amax, fabsf(v[q]));
    // floor(log2 amax) is the exponent field less 127 for a normal amax; a
    // zero or subnormal amax clamps to the smallest scale
    const int ef = (int)(__float_as_uint(amax) >> 23);
    const int shared = ef == 0 ? -127 : max(ef - 127 - 2, -127);
    uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < kMxBlock; ++q) word[q >> 3] |= e2m1_encode(ldexpf(v[q], -shared)) << (4 * (q & 7));
    *(uint4*)(codes + gr * (C / 2) + j * 16) = make_uint4(word[0], word[1], word[2], word[3]);
    scales[(g * nbr + j) * (long)R + r] = (uint8_t)(shared + 127);
  }
}

hipError_t launch_quantize_mxfp4(const void* w, int bf16, int G, int R, int C, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s) {
  const long n = (long)G * R * (C / kMxBlock);
  if (n <= 0) return hipSuccess;
  long grid = (n + 255) / 256;
  if (grid > 65536) grid = 65536;
  if (bf16)
    hipLaunchKernelGGL(quantize_mxfp4_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, w, G, R, C, codes, scales);
  else
    hipLaunchKernelGGL(quantize_mxfp4_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, w, G, R, C, codes,
                       scales);
  return hipGetLastError();
}

}  // namespace moe
