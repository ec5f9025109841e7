// Router: fp32 logits and the group-limited sigmoid top-k.
//
// Logits z = x W_r^T are fp32 ("NemotronH", "Arithmetic").  For bf16 x the
// fp32 weight is split into three bf16 planes hi + mid + lo that sum to W_r
// exactly (each plane keeps the next 8 significant bits), so the product
// x * W_r = x*hi + x*mid + x*lo is formed from exact bf16 x bf16 products on
// MFMA with fp32 accumulation: fp32 logits at matrix-core speed.  The three
// planes are stored K-concatenated ([E][3d]) and the GEMM walks K = 3d
// against x with period d, split over K so the short [T, E] output still
// fills the chip; the route kernel sums the split partials in a fixed order.
//
// Route ("Nemotron is not one circuit", "The Router Is A Deterministic
// Algorithm" / "The C Kernel Contract"): one wave per token row; the row's
// E corrected scores live E/64 per lane; groups scored by their top-2 sum,
// the best topk_group groups kept, then K rounds of a wave-wide maximum over
// 32-bit order-preserving score keys, the lowest lane (and within it the
// lowest slot) holding the maximum winning, so equal scores resolve to the
// lower id; weights from the uncorrected sigmoid, normalised and scaled.
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// W_r -> three bf16 planes
// ---------------------------------------------------------------------------
__global__ void split_router_weight_kernel(const float* __restrict__ w, long n, int d, int dp,
                                           uint16_t* __restrict__ w3) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const long e = i / dp, k = i - e * dp;
    uint32_t hi = 0, mid = 0, lo = 0;
    if (k < d) {
      const float v = w[e * d + k];
      hi = f32_to_bf16(v);
      const float r1 = v - bf16_to_f32(hi);  // exact: v and hi agree in their leading bits
      mid = f32_to_bf16(r1);
      const float r2 = r1 - bf16_to_f32(mid);
      lo = f32_to_bf16(r2);  // r2 has at most 8 significant bits left: exact
    }
    uint16_t* row = w3 + e * 3 * (long)dp;
    row[k] = (uint16_t)hi;
    row[dp + k] = (uint16_t)mid;
    row[2 * (long)dp + k] = (uint16_t)lo;
  }
}

hipError_t launch_split_router_weight(const float* w, int E, int d, uint16_t* w3, hipStream_t s) {
  const int dp = router_plane_width(d);
  const long n = (long)E * dp;
  int grid = (int)((n + 255) / 256);
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(split_router_weight_kernel, dim3(grid), dim3(256), 0, s, w, n, d, dp, w3);
  return hipGetLastError();
}

int router_bf16_splits(int T, int d, int E) {
  const int tiles = ceil_div(T, kDenseChunkRows) * ceil_div(E, kDenseTileN);
  const int nk = 3 * router_plane_width(d) / 64;
  int S = ceil_div(512, tiles);  // aim for two workgroups per CU
  if (S > nk / 2) S = nk / 2;
  if (S < 1) S = 1;
  return S;
}

hipError_t launch_router_gemm_bf16x3(const uint16_t* x, int T, int d, const uint16_t* w3, int E,
                                     float* partials, int S, hipStream_t s) {
  const int dp = router_plane_width(d);
  GemmArgs a = {};
  a.E = 0;
  a.M_s = T;
  a.A_s = x;
  a.lda_s = d;
  a.B_s = w3;
  a.ldb_s = 3L * dp;
  a.N_s = E;
  a.Kd_s = 3 * dp;
  a.C_s = partials;
  a.ldc_s = E;
  a.c_s_f32 = 1;
  a.ksplit = S;
  a.split_stride = (long)T * E;
  a.a_period = dp;
  a.a_cols = d;
  return launch_gemm(a, 1, B_NK, EPI_STORE, 0, s);
}

hipError_t launch_router_gemm_f32(const void* x, int x_bf16, int T, int d, const float* w, int E,
                                  float* logits, hipStream_t s) {
  GemmArgs a = {};
  a.M_s = T;
  a.A_s = x;
  a.lda_s = d;
  a.B_s = w;
  a.ldb_s = d;
  a.N_s = E;
  a.Kd_s = d;
  a.C_s = logits;
  a.ldc_s = E;
  a.c_s_f32 = 1;
  a.ksplit = 1;
  (void)x_bf16;  // fp32 activations only
  return launch_gemm(a, 0, B_NK, EPI_STORE, 0, s);
}

// ---------------------------------------------------------------------------
// Sum of split-K partials (fixed order)
// ---------------------------------------------------------------------------
__global__ void sum_partials_kernel(const float* __restrict__ p, int S, long n, float* __restrict__ out) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    float z = p[i];
    for (int k = 1; k < S; ++k) z += p[k * n + i];
    out[i] = z;
  }
}

hipError_t launch_sum_partials(const float* partials, int S, long n, float* out, hipStream_t s) {
  int grid = (int)((n + 255) / 256);
  if (grid > 4096) grid = 4096;
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(sum_partials_kernel, dim3(grid), dim3(256), 0, s, partials, S, n, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Route
// ---------------------------------------------------------------------------
constexpr int kRouteRows = 4;  // rows (waves) per workgroup

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int S,
                                                    long sstride, const float* __restrict__ bias,
                                                    int T, int E, int K, int n_group,
                                                    int topk_group, int norm, float rsf,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ wts) {
  __shared__ float s_sig[kRouteRows][VPL * 64];
  __shared__ float s_cor[kRouteRows][VPL * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kRouteRows + wave;
  const bool valid = t < T;
  int id;
  float w;
  route_row<VPL>(logits, S, sstride, bias, t, valid, E, K, n_group, topk_group, norm, rsf, s_sig[wave],
                 s_cor[wave], lane, &id, &w);
  if (valid && lane < K) {
    ids[(long)t * K + lane] = id;
    wts[(long)t * K + lane] = w;
  }
}

hipError_t launch_route(const float* logits, int S, const float* bias, int T, int E, int K,
                        int n_group, int topk_group, int norm, float rsf, int32_t* ids,
                        float* weights, hipStream_t s) {
  const int vpl = ceil_div(E, 64);
  dim3 grid(ceil_div(T, kRouteRows)), block(64 * kRouteRows);
  const long sstride = (long)T * E;
#define MOE_ROUTE_CASE(V)                                                                    \
  if (vpl <= V) {                                                                            \
    hipLaunchKernelGGL((route_kernel<V>), grid, block, 0, s, logits, S, sstride, bias, T, E, \
                       K, n_group, topk_group, norm, rsf, ids, weights);                     \
    return hipGetLastError();                                                                \
  }
  MOE_ROUTE_CASE(1)
  MOE_ROUTE_CASE(2)
  MOE_ROUTE_CASE(4)
  MOE_ROUTE_CASE(8)
  MOE_ROUTE_CASE(16)
#undef MOE_ROUTE_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
