// Backward pass of the routed ReLU^2 layer (gradients of a loss through the
// layer output Y): the kernels around the grouped GEMMs.  The steps follow
// "M6.1 - Routed Capacity", 0x06F: the combine adjoint is a broadcast and a
// dot product (0x06F.2), the gates' Jacobian couples a token's routes
// (0x06F.3, here for normalised sigmoid scores), the router projection
// returns G_Z^T x and G_Z W_r (0x06F.4), the gather adjoint is an add into
// the token's row (0x06F.6).  All sums run in a fixed order (no atomics).
#include "moe_internal.h"

namespace moe {

namespace {
constexpr int kBwdThreads = 256;
}  // namespace

// Per token t (one workgroup): q_k = <dY_t, U_{pos_k}> for its accepted
// routes (0 for a dropped one), then with s_k = sigmoid(z_{t, id_k}) and
// g_k the forward's gate weights: normalised, dL/ds_k = (rsf q_k -
// sum_j g_j q_j) / sum_j s_j; otherwise rsf q_k; dz_k = dL/ds_k s_k (1 - s_k).
// Writes dz [T][K] (fp32) and the gated rows dU[pos_k] = bf16(g_k dY_t).
__global__ __launch_bounds__(kBwdThreads) void gate_grad_kernel(
    const uint16_t* __restrict__ dy, const float* __restrict__ U, const float* __restrict__ logits, int S,
    long sstride, const int32_t* __restrict__ ids, const float* __restrict__ gates,
    const int32_t* __restrict__ rpos, int E, int K, int d, int norm, float rsf, float* __restrict__ dz,
    uint16_t* __restrict__ dU) {
  __shared__ float s_q[MOE_MAX_TOPK];
  __shared__ float s_s[MOE_MAX_TOPK];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t* dyr = dy + (long)t * d;
  // the selected experts' sigmoid scores, thread k summing route k's split
  // partials (issued before the row work, so their latency overlaps it)
  if (tid < K) {
    const long idx = (long)t * E + ids[(long)t * K + tid];
    float z = logits[idx];
#pragma unroll 4
    for (int p = 1; p < S; ++p) z += logits[p * sstride + idx];
    s_s[tid] = 1.0f / (1.0f + expf(-z));
  }
  // one wave per route (routes k = wave, wave + 4, ...): its dot product and
  // its gated row
  for (int k = wave; k < K; k += kBwdThreads / 64) {
    const int pos = rpos[(long)t * K + k];
    float acc = 0.0f;
    if (pos >= 0) {
      const float* ur = U + (long)pos * d;
      const float g = gates[(long)t * K + k];
      uint16_t* out = dU + (long)pos * d;
      for (int c = lane * 8; c < d; c += 64 * 8) {
        const uint4 a = *(const uint4*)(dyr + c);
        const float4 b0 = *(const float4*)(ur + c), b1 = *(const float4*)(ur + c + 4);
        const uint32_t ua[4] = {a.x, a.y, a.z, a.w};
        const float ub[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = bf16_to_f32(ua[q] & 0xffffu), hi = bf16_to_f32(ua[q] >> 16);
          acc = fmaf(lo, ub[2 * q], acc);
          acc = fmaf(hi, ub[2 * q + 1], acc);
          o[q] = pack_bf16x2(g * lo, g * hi);
        }
        *(uint4*)(out + c) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) s_q[k] = acc;
  }
  __syncthreads();
  if (tid < K) {
    const int k = tid;
    float ssum = 0.0f, gq = 0.0f, s_me = 0.0f;
    for (int j = 0; j < K; ++j) {
      const float sj = s_s[j];
      ssum += sj;
      gq += gates[(long)t * K + j] * s_q[j];
      if (j == k) s_me = sj;
    }
    const float ds = norm ? (rsf * s_q[k] - gq) / ssum : rsf * s_q[k];
    dz[(long)t * K + k] = ds * s_me * (1.0f - s_me);
  }
}

hipError_t launch_gate_grad(const uint16_t* dy, const float* U, const float* logits, int S, long sstride,
                            const int32_t* ids, const float* gates, const int32_t* rpos, int T, int E, int K, int d,
                            int norm, float rsf, float* dz, uint16_t* dU, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(gate_grad_kernel, dim3(T), dim3(kBwdThreads), 0, s, dy, U, logits, S, sstride, ids, gates,
                     rpos, E, K, d, norm, rsf, dz, dU);
  return hipGetLastError();
}

// dW_r[e][c] = sum over the routes of expert e (every selected route, also
// a dropped one) of dz_route x[token][c], fp32.  A lane owns 8 columns; the
// 4 waves take the expert's routes in 4 contiguous quarters (each in route
// order) and the quarters are added in wave order, so the sum is
// deterministic.  Grid: experts x column blocks of 512.
__global__ __launch_bounds__(kBwdThreads) void router_grad_kernel(const uint16_t* __restrict__ x, int d, int K,
                                                                  const int32_t* __restrict__ offsets,
                                                                  const int32_t* __restrict__ route_src,
                                                                  const float* __restrict__ dz,
                                                                  float* __restrict__ dw) {
  __shared__ float s_part[kBwdThreads / 64][512];
  const int e = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.y * 512 + lane * 8;
  const int a = offsets[e], b = offsets[e + 1];
  const int per = (b - a + 3) / 4;
  const int j0 = a + wave * per, j1 = min(b, j0 + per);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c < d) {
#pragma unroll 4
    for (int j = j0; j < j1; ++j) {
      const int r = route_src[j];
      const float g = dz[r];
      const uint4 v = *(const uint4*)(x + (long)(r / K) * d + c);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(g, bf16_to_f32(u[q] & 0xffffu), acc[2 * q]);
        acc[2 * q + 1] = fmaf(g, bf16_to_f32(u[q] >> 16), acc[2 * q + 1]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) s_part[wave][lane * 8 + q] = acc[q];
  __syncthreads();
  if (wave != 0 || c >= d) return;
  float o[8];
#pragma unroll
  for (int q = 0; q < 8; ++q)
    o[q] = ((s_part[0][lane * 8 + q] + s_part[1][lane * 8 + q]) + s_part[2][lane * 8 + q]) + s_part[3][lane * 8 + q];
  float* po = dw + (long)e * d + c;
  *(float4*)po = make_float4(o[0], o[1], o[2], o[3]);
  *(float4*)(po + 4) = make_float4(o[4], o[5], o[6], o[7]);
}

hipError_t launch_router_grad(const uint16_t* x, int d, int K, int E, const int32_t* offsets,
                              const int32_t* route_src, const float* dz, float* dw, hipStream_t s) {
  if (E <= 0 || d <= 0) return hipSuccess;
  hipLaunchKernelGGL(router_grad_kernel, dim3(E, ceil_div(d, 512)), dim3(kBwdThreads), 0, s, x, d, K,
                     offsets, route_src, dz, dw);
  return hipGetLastError();
}

// dx[t][c] = round(dx_s[t][c] + dx_s2[t][c] + sum over the accepted routes
// in ascending expert id of dxp[pos][c] + sum_k dz[t][k] W_r[id_k][c]): the
// gather adjoint (an add per route), the shared expert's and the router's
// paths, and a second whole-row term (a latent layer's dx_lat W_lin).  Any
// of dx_s, dx_s2, dxp and w_router may be NULL (its term left out: a
// latent layer sums its route rows, L wide, in a call of their own).  With
// dx32 the fp32 sum is stored unrounded there instead (the input of the
// fused front's backward).  A thread owns 4 columns.  Grid: tokens x column
// blocks of 1024.
__global__ __launch_bounds__(kBwdThreads) void dx_combine_kernel(const float* __restrict__ dxp,
                                                                 const float* __restrict__ dx_s,
                                                                 const float* __restrict__ dx_s2,
                                                                 const float* __restrict__ w_router,
                                                                 const int32_t* __restrict__ ids,
                                                                 const int32_t* __restrict__ rpos,
                                                                 const float* __restrict__ dz, int K, int d,
                                                                 uint16_t* __restrict__ dx,
                                                                 float* __restrict__ dx32) {
  __shared__ int s_id[MOE_MAX_TOPK], s_pos[MOE_MAX_TOPK];
  __shared__ float s_dz[MOE_MAX_TOPK];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < 64) {
    const int k = tid;
    const int myid = k < K ? ids[(long)t * K + k] : 0x7fffffff;
    int rank = 0;
    for (int j = 0; j < K; ++j) rank += __shfl(myid, j, 64) < myid;
    if (k < K) {
      s_id[rank] = myid;
      s_pos[rank] = rpos[(long)t * K + k];
      s_dz[rank] = dz[(long)t * K + k];
    }
  }
  __syncthreads();
  const int c = blockIdx.y * (kBwdThreads * 4) + tid * 4;
  if (c >= d) return;
  float4 acc = dx_s ? *(const float4*)(dx_s + (long)t * d + c) : make_float4(0, 0, 0, 0);
  if (dx_s2) {
    const float4 v = *(const float4*)(dx_s2 + (long)t * d + c);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  // the rows are loaded 8 at a time into registers, then added in route
  // order (a dropped route adds nothing)
  constexpr int kB = 8;
  if (dxp)
    for (int r0 = 0; r0 < K; r0 += kB) {
      float4 v[kB];
#pragma unroll
      for (int i = 0; i < kB; ++i)
        if (r0 + i < K && s_pos[r0 + i] >= 0) v[i] = *(const float4*)(dxp + (long)s_pos[r0 + i] * d + c);
#pragma unroll
      for (int i = 0; i < kB; ++i)
        if (r0 + i < K && s_pos[r0 + i] >= 0) {
          acc.x += v[i].x; acc.y += v[i].y; acc.z += v[i].z; acc.w += v[i].w;
        }
    }
  if (w_router)
    for (int r0 = 0; r0 < K; r0 += kB) {
      float4 v[kB];
#pragma unroll
      for (int i = 0; i < kB; ++i)
        if (r0 + i < K) v[i] = *(const float4*)(w_router + (long)s_id[r0 + i] * d + c);
#pragma unroll
      for (int i = 0; i < kB; ++i)
        if (r0 + i < K) {
          const float g = s_dz[r0 + i];
          acc.x = fmaf(g, v[i].x, acc.x); acc.y = fmaf(g, v[i].y, acc.y);
          acc.z = fmaf(g, v[i].z, acc.z); acc.w = fmaf(g, v[i].w, acc.w);
        }
    }
  if (dx32)
    *(float4*)(dx32 + (long)t * d + c) = acc;  // unrounded, for the fused front's backward
  else
    *(uint2*)(dx + (long)t * d + c) = make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
}

hipError_t launch_dx_combine(const float* dxp, const float* dx_s, const float* dx_s2, const float* w_router,
                             const int32_t* ids, const int32_t* rpos, const float* dz, int T, int K, int d,
                             uint16_t* dx, float* dx32, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(dx_combine_kernel, dim3(T, ceil_div(d, kBwdThreads * 4)), dim3(kBwdThreads), 0, s, dxp, dx_s,
                     dx_s2, w_router, ids, rpos, dz, K, d, dx, dx32);
  return hipGetLastError();
}

// Column maps of the transposed operands of the weight-gradient GEMMs: each
// expert's rows padded to a multiple of 8 columns.  koff[e] = sum over e' < e
// of ceil8(count_e') (koff[E] the total); for padded column pc of expert e,
// row_of[pc] = the packed row (offsets[e] + pc - koff[e]) and tok_of[pc] =
// its token (route_src / K), or -1 in the padding.  Each workgroup scans the
// padded counts itself (E <= 1024: one thread per expert) and maps its 1024
// columns; workgroup 0 writes koff.
__global__ __launch_bounds__(1024) void wgrad_map_kernel(const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ route_src, int E, int K,
                                                         int Rp, int32_t* __restrict__ koff,
                                                         int32_t* __restrict__ row_of,
                                                         int32_t* __restrict__ tok_of) {
  __shared__ int s_koff[MOE_MAX_EXPERTS + 1];
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_scan[MOE_MAX_EXPERTS];
  const int tid = threadIdx.x;
  for (int e = tid; e <= E; e += blockDim.x) s_off[e] = offsets[e];
  __syncthreads();
  // inclusive scan of the padded counts (Hillis-Steele over 1024 slots)
  int v = tid < E ? (s_off[tid + 1] - s_off[tid] + 7) & ~7 : 0;
  for (int o = 1; o < MOE_MAX_EXPERTS; o <<= 1) {
    s_scan[tid] = v;
    __syncthreads();
    if (tid >= o) v += s_scan[tid - o];
    __syncthreads();
  }
  if (tid < E) s_koff[tid + 1] = v;
  if (tid == 0) s_koff[0] = 0;
  __syncthreads();
  if (blockIdx.x == 0)
    for (int e = tid; e <= E; e += blockDim.x) koff[e] = s_koff[e];
  const int pc = blockIdx.x * blockDim.x + tid;
  if (pc >= Rp) return;
  if (pc >= s_koff[E]) {
    row_of[pc] = -1;
    tok_of[pc] = -1;
    return;
  }
  // expert of padded column pc: the last e with koff[e] <= pc
  int lo = 0, hi = E;  // invariant: s_koff[lo] <= pc < s_koff[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_koff[mid] <= pc) lo = mid; else hi = mid;
  }
  const int j = s_off[lo] + (pc - s_koff[lo]);
  const bool in = j < s_off[lo + 1];
  row_of[pc] = in ? j : -1;
  tok_of[pc] = in ? route_src[j] / K : -1;
}

hipError_t launch_wgrad_map(const int32_t* offsets, const int32_t* route_src, int E, int K, int Rp, int32_t* koff,
                            int32_t* row_of, int32_t* tok_of, hipStream_t s) {
  static_assert(MOE_MAX_EXPERTS <= 1024, "one scan thread per expert");
  hipLaunchKernelGGL(wgrad_map_kernel, dim3(ceil_div(Rp > 0 ? Rp : 1, 1024)), dim3(1024), 0, s, offsets, route_src,
                     E, K, Rp, koff, row_of, tok_of);
  return hipGetLastError();
}

// out[c][pc] = in[src(pc)][c] (bf16; src(pc) = map[pc], or pc itself when
// map is NULL and pc < nsrc; zero for -1 / past nsrc).  in: [*][C] with row
// stride ldi; out: [C][ncol] with row stride ldo.  64 x 64 tiles through
// LDS, read and written 16 bytes (8 elements) per thread: a source row piece
// of 8 columns in, an output row piece of 8 padded columns out.  C and ncol
// are multiples of 8 and the row strides keep 16-byte alignment.
// Grid: (ceil(ncol / 64), ceil(C / 64)).
__global__ __launch_bounds__(256) void transpose_rows_kernel(const uint16_t* __restrict__ in, long ldi, int C,
                                                             const int32_t* __restrict__ map, int nsrc, int ncol,
                                                             uint16_t* __restrict__ out, long ldo) {
  __shared__ uint16_t tile[64][64 + 2];  // [pc][c]
  const int pc0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int i = (tid >> 3) + it * 32, q = (tid & 7) * 8;  // row pc0 + i, columns c0 + q .. + 7
    const int pc = pc0 + i, c = c0 + q;
    int src = -1;
    if (pc < ncol) src = map ? map[pc] : (pc < nsrc ? pc : -1);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (src >= 0 && c < C) v = *(const uint4*)(in + (long)src * ldi + c);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[i][q + 2 * e] = (uint16_t)(u[e] & 0xffffu);
      tile[i][q + 2 * e + 1] = (uint16_t)(u[e] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int j = (tid >> 3) + it * 32, q = (tid & 7) * 8;  // output row c0 + j, columns pc0 + q .. + 7
    const int c = c0 + j, pc = pc0 + q;
    if (c >= C || pc >= ncol) continue;
    uint32_t u[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = (uint32_t)tile[q + 2 * e][j] | ((uint32_t)tile[q + 2 * e + 1][j] << 16);
    *(uint4*)(out + (long)c * ldo + pc) = make_uint4(u[0], u[1], u[2], u[3]);
  }
}

hipError_t launch_transpose_rows(const uint16_t* in, long ldi, int C, const int32_t* map, int nsrc, int ncol,
                                 uint16_t* out, long ldo, hipStream_t s) {
  if (ncol <= 0 || C <= 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_rows_kernel, dim3(ceil_div(ncol, 64), ceil_div(C, 64)), dim3(256), 0, s, in, ldi, C,
                     map, nsrc, ncol, out, ldo);
  return hipGetLastError();
}

}  // namespace moe
