// Weighted combine back to token rows ("M6.1 - Routed Capacity", 0x05B:
// Y_t = sum of the gated packed rows of token t; 0x05E: an add, never an
// overwrite; "NemotronH", "Arithmetic": the weighted sum in fp32 in
// ascending expert id, one rounding).
//
// One workgroup per token row; each thread owns 8 consecutive columns (one
// 16-byte bf16 chunk) and walks the token's K routes in ascending expert id,
// so the summation order is fixed and no atomics are needed.  A route whose
// packed row is -1 overflowed a fixed capacity and is skipped (fixed drop,
// "M6.1 - Routed Capacity", 0x05F: the other gates are not renormalised).  The shared
// expert's fp32 row and then the residual source (the old output, or the
// layer's input hidden state) join the same fp32 sum before the single
// rounding.
#include "moe_internal.h"

namespace moe {

// YB: packed rows in bf16 (else fp32); BF16: output in bf16 (else fp32).
template <bool YB, bool BF16>
__global__ void combine_kernel(const void* __restrict__ y, const float* __restrict__ w,
                               const int32_t* __restrict__ ids, const int32_t* __restrict__ rpos,
                               const float* __restrict__ ys, int T, int K, int d,
                               const void* resid, void* __restrict__ out) {
  __shared__ int s_pos[MOE_MAX_TOPK];
  __shared__ float s_w[MOE_MAX_TOPK];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < 64) {
    // rank of slot k among the token's (distinct) expert ids
    const int k = tid;
    const int myid = k < K ? ids[(long)t * K + k] : 0x7fffffff;
    int rank = 0;
    for (int j = 0; j < K; ++j) {
      const int o = __shfl(myid, j, 64);
      rank += o < myid;
    }
    if (k < K) {
      s_pos[rank] = rpos[(long)t * K + k];
      s_w[rank] = w[(long)t * K + k];
    }
  }
  __syncthreads();
  const int c = tid;
  if (c * 8 >= d) return;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
  for (int r = 0; r < K; ++r) {
    const float g = s_w[r];
    const long row = s_pos[r];
    if (row < 0) continue;
    if (YB) {
      const uint4 v = *(const uint4*)((const uint16_t*)y + row * d + c * 8);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(g, bf16_to_f32(u[q] & 0xffffu), acc[2 * q]);
        acc[2 * q + 1] = fmaf(g, bf16_to_f32(u[q] >> 16), acc[2 * q + 1]);
      }
    } else {
      const float4* p = (const float4*)((const float*)y + row * d + c * 8);
      const float4 a = p[0], b = p[1];
      const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = fmaf(g, f[q], acc[q]);
    }
  }
  const long o = (long)t * d + c * 8;
  if (ys) {
    const float4 a = *(const float4*)(ys + o), b = *(const float4*)(ys + o + 4);
    acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
    acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
  }
  if (BF16) {
    uint16_t* po = (uint16_t*)out + o;
    if (resid) {
      const uint4 v = *(const uint4*)((const uint16_t*)resid + o);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_to_f32(u[q] & 0xffffu);
        acc[2 * q + 1] += bf16_to_f32(u[q] >> 16);
      }
    }
    uint4 r;
    r.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
    r.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
    r.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
    r.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
    *(uint4*)po = r;
  } else {
    float* po = (float*)out + o;
    if (resid) {
      const float* pr = (const float*)resid + o;
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += pr[q];
    }
    *(float4*)po = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *(float4*)(po + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

hipError_t launch_combine(const void* y_packed, int act_bf16, const float* weights,
                          const int32_t* ids, const int32_t* route_pos, const float* y_shared,
                          int T, int K, int d, const void* resid, void* out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  int threads = ceil_div(d / 8, 64) * 64;
  if (threads < 64) threads = 64;
  if (threads > 1024) return hipErrorInvalidValue;
  if (act_bf16)
    hipLaunchKernelGGL((combine_kernel<true, true>), dim3(T), dim3(threads), 0, s, y_packed, weights, ids,
                       route_pos, y_shared, T, K, d, resid, out);
  else
    hipLaunchKernelGGL((combine_kernel<false, false>), dim3(T), dim3(threads), 0, s, y_packed, weights, ids,
                       route_pos, y_shared, T, K, d, resid, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-K reduction of a dense GEMM: the S fp32 slices summed in order, then
// the addend and the residual source, rounded once (the order and the one
// rounding of the unsplit GEMM's epilogue).  A thread owns 4 columns.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ part, int S, long stride,
                                                            int rows, int N, const float* __restrict__ addend,
                                                            long ld_add, const void* resid, void* out) {
  const long n4 = (long)rows * (N / 4);
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (long)gridDim.x * blockDim.x) {
    const long r = i / (N / 4);
    const int c = (int)(i - r * (N / 4)) * 4;
    const long o = r * N + c;
    float4 a = *(const float4*)(part + o);
    for (int k = 1; k < S; ++k) {
      const float4 b = *(const float4*)(part + k * stride + o);
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    if (addend) {
      const float4 b = *(const float4*)(addend + r * ld_add + c);
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    if (BF16) {
      if (resid) {
        const uint2 v = *(const uint2*)((const uint16_t*)resid + o);
        a.x += bf16_to_f32(v.x & 0xffffu); a.y += bf16_to_f32(v.x >> 16);
        a.z += bf16_to_f32(v.y & 0xffffu); a.w += bf16_to_f32(v.y >> 16);
      }
      *(uint2*)((uint16_t*)out + o) = make_uint2(f32_to_bf16(a.x) | (f32_to_bf16(a.y) << 16),
                                                 f32_to_bf16(a.z) | (f32_to_bf16(a.w) << 16));
    } else {
      if (resid) {
        const float4 b = *(const float4*)((const float*)resid + o);
        a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
      }
      *(float4*)((float*)out + o) = a;
    }
  }
}

hipError_t launch_reduce_splits(const float* part, int S, long split_stride, int rows, int N, const float* addend,
                                long ld_add, const void* resid, void* out, int out_bf16, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (N % 4 || S < 1) return hipErrorInvalidValue;
  const long n4 = (long)rows * (N / 4);
  long grid = (n4 + 255) / 256;
  if (grid > 8192) grid = 8192;
  if (out_bf16)
    hipLaunchKernelGGL(reduce_splits_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, part, S, split_stride, rows,
                       N, addend, ld_add, resid, out);
  else
    hipLaunchKernelGGL(reduce_splits_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, part, S, split_stride,
                       rows, N, addend, ld_add, resid, out);
  return hipGetLastError();
}

hipError_t launch_combine_y32(const float* y_packed, const float* weights, const int32_t* ids,
                              const int32_t* route_pos, const float* y_shared, int T, int K, int d,
                              const void* resid, void* out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  int threads = ceil_div(d / 8, 64) * 64;
  if (threads < 64) threads = 64;
  if (threads > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL((combine_kernel<false, true>), dim3(T), dim3(threads), 0, s, y_packed, weights, ids, route_pos,
                     y_shared, T, K, d, resid, out);
  return hipGetLastError();
}

}  // namespace moe
