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

// ---------------------------------------------------------------------------
// Backward of the fused front (bf16 rows): with r = 1 / sqrt(mean(h^2) +
// eps) computed exactly as the forward computes it, n = h r and dn = dx w
// (dx the fp32 gradient reaching the normed rows):
//   dH = dY + (dn - n mean(n dn)) r    (rounded once to bf16; dY is the
//        residual's path, out = Y + H),
//   dw_norm = sum over rows of dx n     (rmsnorm_dw_*: partial sums over
//        blocks of 64 rows, then the blocks in order).
// One wave per row; the row of h stays in registers, dx and w are read
// twice.  The sum of n dn has the forward's fixed order (lane-local chunks,
// then halving folds).  r of each row goes to r_out for the weight gradient.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const uint16_t* __restrict__ h,
                                                          const uint16_t* __restrict__ w, float eps, int T, int d,
                                                          const float* __restrict__ dx,
                                                          const uint16_t* __restrict__ dy,
                                                          uint16_t* __restrict__ dh, float* __restrict__ r_out) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const int nch = d / 8;
  const long base = (long)row * d;
  uint4 keep[kNormChunks];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kNormChunks; ++i) {
    const int c = lane + 64 * i;
    keep[i] = c < nch ? *(const uint4*)(h + base + c * 8) : make_uint4(0, 0, 0, 0);
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
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s = s + __shfl_xor(s, off, 64);
  const float ms = s / (float)d;
  const float r = 1.0f / sqrtf(ms + eps);
  if (lane == 0) r_out[row] = r;
  // pass 1: sum of n dn
  float s2 = 0.0f;
#pragma unroll
  for (int i = 0; i < kNormChunks; ++i) {
    const int c = lane + 64 * i;
    if (c >= nch) break;
    float v[8], g[8], e[8];
    unpack8(keep[i], v);
    load8<true>(w, (long)c * 8, g);
    load8<false>(dx, base + c * 8, e);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float n = v[q] * r, dn = e[q] * g[q];
      const float t = n * dn;
      s2 = s2 + t;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s2 = s2 + __shfl_xor(s2, off, 64);
  const float m2 = s2 / (float)d;
  // pass 2: dH
#pragma unroll
  for (int i = 0; i < kNormChunks; ++i) {
    const int c = lane + 64 * i;
    if (c >= nch) break;
    float v[8], g[8], e[8], y[8], o[8];
    unpack8(keep[i], v);
    load8<true>(w, (long)c * 8, g);
    load8<false>(dx, base + c * 8, e);
    load8<true>(dy, base + c * 8, y);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float n = v[q] * r, dn = e[q] * g[q];
      const float nm = n * m2;
      const float t = (dn - nm) * r;
      o[q] = y[q] + t;
    }
    *(uint4*)(dh + base + c * 8) = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                              pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
  }
}

constexpr int kDwRows = 64;  // rows per partial sum of the norm weight's gradient

// part[b][j] = sum over rows t of block b (ascending) of dx[t][j] (h[t][j] r[t]).
__global__ __launch_bounds__(256) void rmsnorm_dw_part_kernel(const uint16_t* __restrict__ h, const float* __restrict__ dx,
                                                              const float* __restrict__ r, int T, int d,
                                                              float* __restrict__ part) {
#pragma clang fp contract(off)
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d) return;
  const int t0 = blockIdx.y * kDwRows, t1 = min(T, t0 + kDwRows);
  float acc = 0.0f;
  for (int t = t0; t < t1; ++t) {
    const float n = bf16_to_f32(h[(long)t * d + j]) * r[t];
    const float v = dx[(long)t * d + j] * n;
    acc = acc + v;
  }
  part[(long)blockIdx.y * d + j] = acc;
}

// dw[j] = sum over the blocks in order of part[b][j].
__global__ __launch_bounds__(256) void rmsnorm_dw_sum_kernel(const float* __restrict__ part, int nb, int d,
                                                             float* __restrict__ dw) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= d) return;
  float acc = 0.0f;
  for (int b = 0; b < nb; ++b) acc += part[(long)b * d + j];
  dw[j] = acc;
}

int rmsnorm_dw_blocks(int T) { return ceil_div(T > 0 ? T : 1, kDwRows); }

hipError_t launch_rmsnorm_bwd(const uint16_t* h, const uint16_t* w, float eps, int T, int d, const float* dx,
                              const uint16_t* dy, uint16_t* dh, float* dw, float* r_buf, float* part,
                              hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (d > kNormChunks * 64 * 8 || d % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rmsnorm_bwd_kernel, dim3(ceil_div(T, 4)), dim3(256), 0, s, h, w, eps, T, d, dx, dy, dh, r_buf);
  const int nb = rmsnorm_dw_blocks(T);
  hipLaunchKernelGGL(rmsnorm_dw_part_kernel, dim3(ceil_div(d, 256), nb), dim3(256), 0, s, h, dx, r_buf, T, d, part);
  hipLaunchKernelGGL(rmsnorm_dw_sum_kernel, dim3(ceil_div(d, 256)), dim3(256), 0, s, part, nb, d, dw);
  return hipGetLastError();
}

}  // namespace moe
