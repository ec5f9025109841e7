// RMSNorm in front of the layer ("NemotronH", "Arithmetic": the RMS norm in
// fp32 times the plain weight; "Nemotron is not one circuit", "The Four
// Layer Kinds CKE Must Preserve": RMSNorm -> router -> ... -> residual).
//
// One wave per row; a bf16 row stays in registers between the sum of squares
// and the scaling (at most 16 chunks of 8 per lane: d <= 8192), an fp32 row
// is read again.  The fp32 sum of squares has a fixed order: lane j owns
// the 8-element chunks j, j + 64, j + 128, ... and adds their squares in
// element order; the 64 lane sums are then added in halving folds (lane j +
// lane j + 32, then + 16, ...), which the xor butterfly computes on every
// lane.  Every product and sum is rounded to fp32 on its own (no fused
// multiply-add), the mean is the sum divided by the width, and 1 / sqrt(mean
// + eps) uses the correctly rounded square root and division, so the
// result, rounded once to the activation dtype, is the same value on any
// run.
#include "moe_internal.h"

namespace moe {

template <bool BF16>
__device__ __forceinline__ void load8(const void* p, long off, float (&v)[8]) {
  if (BF16) {
    const uint4 u = *(const uint4*)((const uint16_t*)p + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16_to_f32(w[q] & 0xffffu);
      v[2 * q + 1] = bf16_to_f32(w[q] >> 16);
    }
  } else {
    const float4 a = *(const float4*)((const float*)p + off), b = *(const float4*)((const float*)p + off + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

constexpr int kNormChunks = 16;  // 8-element chunks per lane kept in registers

__device__ __forceinline__ void unpack8(const uint4 u, float (&v)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = bf16_to_f32(w[q] & 0xffffu);
    v[2 * q + 1] = bf16_to_f32(w[q] >> 16);
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* __restrict__ x, const void* __restrict__ w,
                                                      float eps, int T, int d, void* __restrict__ y) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const int nch = d / 8;
  const long base = (long)row * d;
  float s = 0.0f;
  uint4 keep[BF16 ? kNormChunks : 1];
  if (BF16) {
#pragma unroll
    for (int i = 0; i < kNormChunks; ++i) {
      const int c = lane + 64 * i;
      keep[i] = c < nch ? *(const uint4*)((const uint16_t*)x + base + c * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kNormChunks; ++i) {
      if (lane + 64 * i >= nch) break;
      float v[8];
      unpack8(keep[i], v);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float sq = v[q] * v[q];
        s = s + sq;
      }
    }
  } else {
    for (int c = lane; c < nch; c += 64) {
      float v[8];
      load8<BF16>(x, base + c * 8, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float sq = v[q] * v[q];
        s = s + sq;
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s = s + __shfl_xor(s, off, 64);
  const float ms = s / (float)d;
  const float r = 1.0f / sqrtf(ms + eps);
  // y = (x * r) * w, each product rounded to fp32, then one rounding to dt
  auto emit = [&](int c, const float (&v)[8]) {
    float g[8];
    load8<BF16>(w, (long)c * 8, g);
    float o[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float t = v[q] * r;
      o[q] = t * g[q];
    }
    if (BF16) {
      *(uint4*)((uint16_t*)y + base + c * 8) =
          make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                     pack_bf16x2(o[6], o[7]));
    } else {
      float* py = (float*)y + base + c * 8;
      *(float4*)py = make_float4(o[0], o[1], o[2], o[3]);
      *(float4*)(py + 4) = make_float4(o[4], o[5], o[6], o[7]);
    }
  };
  if (BF16) {
#pragma unroll
    for (int i = 0; i < kNormChunks; ++i) {
      const int c = lane + 64 * i;
      if (c >= nch) break;
      float v[8];
      unpack8(keep[i], v);
      emit(c, v);
    }
  } else {
    for (int c = lane; c < nch; c += 64) {
      float v[8];
      load8<BF16>(x, base + c * 8, v);
      emit(c, v);
    }
  }
}

hipError_t launch_rmsnorm(const void* x, const void* w, float eps, int T, int d, int bf16, void* y,
                          hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (bf16 && d > kNormChunks * 64 * 8) return hipErrorInvalidValue;  // the row must fit the registers
  const dim3 grid(ceil_div(T, 4)), block(256);
  if (bf16)
    hipLaunchKernelGGL(rmsnorm_kernel<true>, grid, block, 0, s, x, w, eps, T, d, y);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<false>, grid, block, 0, s, x, w, eps, T, d, y);
  return hipGetLastError();
}

}  // namespace moe
