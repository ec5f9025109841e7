// Zero-skipping down projection for decode-size batches.
//
// After ReLU^2 many hidden activations are exactly zero, and a zero neuron
// contributes nothing to the down projection, so its weights need not be
// read (the 8 GB Nemotron-3.5-Super write-up, "The engine, step by step",
// item 4).  The down weights are stored neuron-major ([F][d_e]), so each
// skipped neuron is one whole contiguous row of weights never fetched.
//
// live_rows: per expert (and for the shared expert), the ascending list of
// hidden neurons that are non-zero for at least one of its rows, built with
// an ordered wave-ballot compaction; it also counts the exact zeros.
// down_zero_skip: per (expert, 64-column slice), 32 neuron lanes x 8
// column threads stream the live weight rows and accumulate up to 8 rows at
// a time in fp32; the 32 partial sums are added in a fixed order through
// LDS, so the result is deterministic.
#include "moe_internal.h"

namespace moe {

struct ZsGroup {
  long base;
  int M;
  const void* h;
  long ldh;
  int F;
  int32_t* live_idx;
  int32_t* live_cnt;
  const void* w;
  int ncols;
  void* y;
  long ldy;
  int y_f32;
  int zc;  // index of the group's zero counter (0 routed, 2 group 0)
};

template <bool BF16>
__device__ __forceinline__ ZsGroup zs_group(const ZsArgs& z, int g) {
  ZsGroup q;
  if (g < z.E) {
    q.base = z.offsets[g];
    q.M = z.offsets[g + 1] - (int)q.base;
    q.h = z.h;
    q.ldh = z.ldh;
    q.F = z.F;
    q.live_idx = z.live_idx + (long)g * z.F;
    q.live_cnt = z.live_cnt + g;
    const long off = (long)g * z.F * z.d_e;
    q.w = BF16 ? (const void*)((const uint16_t*)z.w + off) : (const void*)((const float*)z.w + off);
    q.ncols = z.d_e;
    q.y = z.y;
    q.ldy = z.ldy;
    q.y_f32 = z.y_f32;
    q.zc = 0;
  } else {
    q.base = 0;
    q.M = z.M_s;
    q.h = z.h_s;
    q.ldh = z.ldh_s;
    q.F = z.F_s;
    q.live_idx = z.live_idx_s;
    q.live_cnt = z.live_cnt_s;
    q.w = z.w_s;
    q.ncols = z.d_s;
    q.y = z.y_s;
    q.ldy = z.ldy_s;
    q.y_f32 = z.y_s_f32;
    q.zc = 2;
  }
  return q;
}

template <bool BF16>
__device__ __forceinline__ bool is_nonzero(const void* h, long idx) {
  if (BF16) return (((const uint16_t*)h)[idx] & 0x7fffu) != 0;
  return ((const float*)h)[idx] != 0.0f;
}

template <bool BF16>
__device__ __forceinline__ float load_act(const void* h, long idx) {
  if (BF16) return bf16_to_f32(((const uint16_t*)h)[idx]);
  return ((const float*)h)[idx];
}

template <bool BF16>
__global__ __launch_bounds__(256) void live_rows_kernel(ZsArgs z) {
  __shared__ int s_wave[4];
  __shared__ unsigned long long s_zero[4];
  const ZsGroup q = zs_group<BF16>(z, blockIdx.x);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  long zeros = 0;
  int cnt = 0;
  if (q.M > 0) {
    for (int fb = 0; fb < q.F; fb += 256) {
      const int f = fb + tid;
      bool live = false;
      if (f < q.F) {
        for (int r = 0; r < q.M; ++r) {
          const bool nz = is_nonzero<BF16>(q.h, (q.base + r) * q.ldh + f);
          live |= nz;
          zeros += nz ? 0 : 1;
        }
      }
      const unsigned long long b = __ballot(live);
      const unsigned long long below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
      const int pre = __popcll(b & below);
      if (lane == 0) s_wave[wave] = __popcll(b);
      __syncthreads();
      int wbase = 0, total = 0;
      for (int w = 0; w < 4; ++w) {
        if (w < wave) wbase += s_wave[w];
        total += s_wave[w];
      }
      if (live) q.live_idx[cnt + wbase + pre] = f;
      cnt += total;
      __syncthreads();
    }
  }
  // block sum of zeros
  unsigned long long zw = zeros;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) zw += __shfl_xor(zw, off, 64);
  if (lane == 0) s_zero[wave] = zw;
  __syncthreads();
  if (tid == 0) {
    *q.live_cnt = cnt;
    if (z.zero_count && q.M > 0) {
      const unsigned long long zt = s_zero[0] + s_zero[1] + s_zero[2] + s_zero[3];
      atomicAdd((unsigned long long*)&z.zero_count[q.zc], zt);
      atomicAdd((unsigned long long*)&z.zero_count[q.zc + 1], (unsigned long long)(q.F - cnt));
    }
  }
}

constexpr int kZsSlice = 64;  // output columns per workgroup
constexpr int kZsRows = 8;    // rows accumulated per pass

template <bool BF16>
__global__ __launch_bounds__(256) void down_zero_skip_kernel(ZsArgs z, int nsl_r, int nsl_s) {
  __shared__ float s_red[32][kZsRows][kZsSlice];
  int g, sl;
  const int nr = z.E * nsl_r;
  if ((int)blockIdx.x < nr) {
    g = blockIdx.x / nsl_r;
    sl = blockIdx.x - g * nsl_r;
  } else {
    g = z.E;
    sl = blockIdx.x - nr;
    if (sl >= nsl_s) return;
  }
  const ZsGroup q = zs_group<BF16>(z, g);
  if (q.M <= 0) return;
  const int tid = threadIdx.x, fl = tid >> 3, cg = tid & 7;
  const int n0 = sl * kZsSlice;
  const int col = n0 + cg * 8;
  const bool colok = col < q.ncols;
  const int nl = *q.live_cnt;
  for (int r0 = 0; r0 < q.M; r0 += kZsRows) {
    const int rows = min(kZsRows, q.M - r0);
    float acc[kZsRows][8];
#pragma unroll
    for (int r = 0; r < kZsRows; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[r][c] = 0.0f;
    for (int i = fl; i < nl; i += 4 * 32) {
      int fs[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) fs[u] = (i + 32 * u < nl) ? q.live_idx[i + 32 * u] : -1;
      float wv[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (fs[u] >= 0 && colok) {
          const long wo = (long)fs[u] * q.ncols + col;
          if (BF16) {
            const uint4 v = *(const uint4*)((const uint16_t*)q.w + wo);
            const uint32_t uu[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              wv[u][2 * c] = bf16_to_f32(uu[c] & 0xffffu);
              wv[u][2 * c + 1] = bf16_to_f32(uu[c] >> 16);
            }
          } else {
            const float4 a = *(const float4*)((const float*)q.w + wo);
            const float4 b = *(const float4*)((const float*)q.w + wo + 4);
            wv[u][0] = a.x; wv[u][1] = a.y; wv[u][2] = a.z; wv[u][3] = a.w;
            wv[u][4] = b.x; wv[u][5] = b.y; wv[u][6] = b.z; wv[u][7] = b.w;
          }
        } else {
#pragma unroll
          for (int c = 0; c < 8; ++c) wv[u][c] = 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (fs[u] < 0) continue;
#pragma unroll
        for (int r = 0; r < kZsRows; ++r) {
          if (r < rows) {
            const float hv = load_act<BF16>(q.h, (q.base + r0 + r) * q.ldh + fs[u]);
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[r][c] = fmaf(hv, wv[u][c], acc[r][c]);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kZsRows; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) s_red[fl][r][cg * 8 + c] = acc[r][c];
    __syncthreads();
    for (int o = tid; o < kZsRows * kZsSlice; o += 256) {
      const int r = o / kZsSlice, cc = o - r * kZsSlice;
      if (r < rows && n0 + cc < q.ncols) {
        float v = 0.0f;
        for (int j = 0; j < 32; ++j) v += s_red[j][r][cc];
        const long yo = (q.base + r0 + r) * q.ldy + n0 + cc;
        if (q.y_f32)
          ((float*)q.y)[yo] = v;
        else
          ((uint16_t*)q.y)[yo] = (uint16_t)f32_to_bf16(v);
      }
    }
    __syncthreads();
  }
}

hipError_t launch_live_rows(const ZsArgs& z, int act_bf16, hipStream_t s) {
  const int groups = z.E + (z.M_s > 0 ? 1 : 0);
  if (groups == 0) return hipSuccess;
  if (act_bf16)
    hipLaunchKernelGGL(live_rows_kernel<true>, dim3(groups), dim3(256), 0, s, z);
  else
    hipLaunchKernelGGL(live_rows_kernel<false>, dim3(groups), dim3(256), 0, s, z);
  return hipGetLastError();
}

hipError_t launch_down_zero_skip(const ZsArgs& z, int act_bf16, hipStream_t s) {
  const int nsl_r = ceil_div(z.d_e, kZsSlice);
  const int nsl_s = z.M_s > 0 ? ceil_div(z.d_s, kZsSlice) : 0;
  const int grid = z.E * nsl_r + nsl_s;
  if (grid == 0) return hipSuccess;
  if (act_bf16)
    hipLaunchKernelGGL(down_zero_skip_kernel<true>, dim3(grid), dim3(256), 0, s, z, nsl_r, nsl_s);
  else
    hipLaunchKernelGGL(down_zero_skip_kernel<false>, dim3(grid), dim3(256), 0, s, z, nsl_r, nsl_s);
  return hipGetLastError();
}

}  // namespace moe
