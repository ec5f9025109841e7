// Dispatch: per-expert histogram, prefix-sum offsets and the expert-major
// permutation of the T*K routes in (expert, token, slot) order ("M6.1 -
// Routed Capacity", 0x05A and 0x05E), plus the tile plans of the grouped
// GEMMs built from the per-expert counts on the device (no host readback).
//
// Tokens are taken 256 per workgroup (a chunk), 64 per wave.  Each wave
// marks, per expert, the lanes (tokens) that chose it with an LDS 64-bit
// atomic OR; OR is order-independent, so the masks -- and every count and
// rank derived from them by popcount -- are deterministic.  A token's rank
// inside its expert is the popcount of the earlier waves' masks plus the
// popcount of its own wave's mask below its lane; adding the chunk's
// running base and the expert's offset gives its packed row.
#include "moe_internal.h"

namespace moe {

constexpr int kDispatchChunk = 256;

size_t dispatch_scratch_bytes(int T, int E) {
  return (size_t)ceil_div(T > 0 ? T : 1, kDispatchChunk) * E * sizeof(int32_t);
}

__device__ __forceinline__ void build_masks(unsigned long long (*masks)[MOE_MAX_EXPERTS],
                                            const int32_t* __restrict__ ids, int T, int K, int E) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += blockDim.x)
#pragma unroll
    for (int w = 0; w < 4; ++w) masks[w][e] = 0ull;
  __syncthreads();
  const long t = (long)blockIdx.x * kDispatchChunk + tid;
  if (t < T)
    for (int k = 0; k < K; ++k) atomicOr(&masks[wave][ids[t * K + k]], 1ull << lane);
  __syncthreads();
}

__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ ids, int T,
                                                             int K, int E,
                                                             int32_t* __restrict__ chunk_counts) {
  __shared__ unsigned long long masks[4][MOE_MAX_EXPERTS];
  build_masks(masks, ids, T, K, E);
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    chunk_counts[(long)blockIdx.x * E + e] =
        __popcll(masks[0][e]) + __popcll(masks[1][e]) + __popcll(masks[2][e]) + __popcll(masks[3][e]);
}

// Exclusive scan of v over the block (blockDim.x <= 1024); returns the
// exclusive prefix of this thread and writes the total to *total.
__device__ int block_exclusive_scan(int v, int* scratch /*[32]*/, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = (blockDim.x + 63) >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      const int s = scratch[w];
      scratch[w] = run;
      run += s;
    }
    scratch[31] = run;
  }
  __syncthreads();
  const int res = scratch[wave] + x - v;
  *total = scratch[31];
  __syncthreads();
  return res;
}

// Tile plans for the up and the down GEMM from per-expert counts in LDS.
__device__ void build_plans(const int* s_count, int E, const PlanOut& P, int* s_gstart,
                            int* scratch) {
  const int tid = threadIdx.x;
  for (int which = 0; which < 2; ++which) {
    const PlanSpec& ps = which == 0 ? P.up : P.down;
    int32_t* plan = which == 0 ? P.plan_up : P.plan_down;
    // group g: 0 = dense group, g >= 1 = expert g-1; E + 1 <= 1025 groups
    int total = 0;
    for (int base = 0; base < E + 1; base += blockDim.x) {
      const int g = base + tid;
      int n = 0;
      if (g == 0)
        n = ceil_div(ps.M_s, kChunkRows) * ps.ntc_s;
      else if (g <= E)
        n = ceil_div(s_count[g - 1], kChunkRows) * ps.ntc_r;
      int seg_total;
      const int ex = block_exclusive_scan(g <= E ? n : 0, scratch, &seg_total);
      if (g <= E) s_gstart[g] = total + ex;
      total += seg_total;
    }
    if (tid == 0) {
      s_gstart[E + 1] = total;
      P.num_tiles[which] = total;
    }
    __syncthreads();
    for (int t = tid; t < total; t += blockDim.x) {
      int lo = 0, hi = E;  // largest g with gstart[g] <= t
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_gstart[mid] <= t)
          lo = mid;
        else
          hi = mid - 1;
      }
      const int g = lo;
      const int l = t - s_gstart[g];
      const int nch = g == 0 ? ceil_div(ps.M_s, kChunkRows) : ceil_div(s_count[g - 1], kChunkRows);
      const int ntc = g == 0 ? ps.ntc_s : ps.ntc_r;
      int ch, nt;
      plan_decode_local(l, nch, ntc, &ch, &nt);
      plan[2 * (long)t] = g;
      plan[2 * (long)t + 1] = (ch << 16) | nt;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(int32_t* __restrict__ chunk_counts, int C,
                                                             int E, int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             PlanOut P, int with_plan) {
  __shared__ int s_count[MOE_MAX_EXPERTS];
  __shared__ int s_gstart[MOE_MAX_EXPERTS + 2];
  __shared__ int scratch[32];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) {
    int run = 0;
    int c = 0;
    for (; c + 8 <= C; c += 8) {
      int v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = chunk_counts[(long)(c + q) * E + e];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        chunk_counts[(long)(c + q) * E + e] = run;
        run += v[q];
      }
    }
    for (; c < C; ++c) {
      const int v = chunk_counts[(long)c * E + e];
      chunk_counts[(long)c * E + e] = run;
      run += v;
    }
    s_count[e] = run;
    counts[e] = run;
  }
  __syncthreads();
  int total = 0;
  for (int base = 0; base < E; base += blockDim.x) {
    const int e = base + tid;
    int seg_total;
    const int ex = block_exclusive_scan(e < E ? s_count[e] : 0, scratch, &seg_total);
    if (e < E) offsets[e] = total + ex;
    total += seg_total;
  }
  if (tid == 0) offsets[E] = total;
  if (with_plan) build_plans(s_count, E, P, s_gstart, scratch);
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(const int32_t* __restrict__ ids, int T,
                                                               int K, int E,
                                                               const int32_t* __restrict__ chunk_base,
                                                               const int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ route_src,
                                                               int32_t* __restrict__ route_pos) {
  __shared__ unsigned long long masks[4][MOE_MAX_EXPERTS];
  build_masks(masks, ids, T, K, E);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long t = (long)blockIdx.x * kDispatchChunk + tid;
  if (t >= T) return;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int k = 0; k < K; ++k) {
    const int e = ids[t * K + k];
    int rank = __popcll(masks[wave][e] & below);
    for (int w = 0; w < wave; ++w) rank += __popcll(masks[w][e]);
    const int pos = offsets[e] + chunk_base[(long)blockIdx.x * E + e] + rank;
    route_src[pos] = (int32_t)(t * K + k);
    route_pos[t * K + k] = pos;
  }
}

// ---------------------------------------------------------------------------
// Fixed capacity ("M6.1 - Routed Capacity", 0x06 and 0x06A): each expert
// keeps the first C of its routes ranked by descending gate, then token,
// then selected slot; the accepted routes keep the (expert, token, slot)
// packed order (0x05E) and an overflowed route gets route_pos = -1.
// One workgroup per expert, over the dropless dispatch of all routes.  The
// rank order is the order of the 64-bit key (~orderable(gate) << 32) | route
// (route = token * K + slot); the C-th smallest key is found by an 8-pass
// radix select (LDS histograms of 8-bit digits), and the routes with keys up
// to it are compacted in packed order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t float_orderable(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kCapThreads = 1024;
constexpr int kCapKeys = 16;  // keys per thread held in registers (routes of one expert up to 16384)

__global__ __launch_bounds__(kCapThreads) void capacity_kernel(const int32_t* __restrict__ counts_all,
                                                              const int32_t* __restrict__ offsets_all,
                                                              const int32_t* __restrict__ src_all,
                                                              const float* __restrict__ gates, int E, int C,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ route_src,
                                                              int32_t* __restrict__ route_pos) {
  __shared__ int scratch[32];
  __shared__ unsigned s_hist[256];
  __shared__ unsigned long long s_prefix, s_thr;
  __shared__ int s_rank, s_bucket;
  const int e = blockIdx.x, tid = threadIdx.x;
  // packed offset of this expert's accepted rows
  int part = 0;
  for (int i = tid; i < e; i += kCapThreads) part += min(counts_all[i], C);
  int off;
  block_exclusive_scan(part, scratch, &off);
  const int n = counts_all[e], base = offsets_all[e], A = min(n, C);
  if (tid == 0) {
    counts[e] = A;
    offsets[e] = off;
    if (e == E - 1) offsets[E] = off + A;
  }
  auto key_of = [&](int j) -> unsigned long long {
    const int32_t r = src_all[base + j];
    return ((unsigned long long)(~float_orderable(gates[r])) << 32) | (uint32_t)r;
  };
  // the expert's keys, thread tid holding rows tid + kCapThreads * i
  const bool cached = n <= kCapThreads * kCapKeys;
  unsigned long long kc[kCapKeys];
#pragma unroll
  for (int i = 0; i < kCapKeys; ++i) {
    const int j = tid + kCapThreads * i;
    kc[i] = (cached && j < n) ? key_of(j) : ~0ull;
  }
  // visit every key of the expert (from registers when cached)
  auto for_keys = [&](auto&& fn) {
    if (cached) {
#pragma unroll
      for (int i = 0; i < kCapKeys; ++i)
        if (tid + kCapThreads * i < n) fn(kc[i]);
    } else {
      for (int j = tid; j < n; j += kCapThreads) fn(key_of(j));
    }
  };
  unsigned long long thr = ~0ull;  // every route fits (with C = 0 none is taken below)
  if (n > C && C > 0) {
    if (tid == 0) {
      s_prefix = 0;
      s_rank = C;  // 1-based rank of the last accepted key among those matching the prefix
      s_thr = ~0ull;
    }
    __syncthreads();
    unsigned long long mask = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kCapThreads) s_hist[i] = 0;
      __syncthreads();
      const unsigned long long pre = s_prefix;
      for_keys([&](unsigned long long k) {
        if ((k & mask) == pre) atomicAdd(&s_hist[(k >> shift) & 255u], 1u);
      });
      __syncthreads();
      // the digit whose bucket holds the wanted rank: a scan over the 256 bins
      const int want = s_rank;
      const unsigned hb = tid < 256 ? s_hist[tid] : 0u;
      int tot;
      const int below = block_exclusive_scan((int)hb, scratch, &tot);
      if (tid < 256 && below < want && want <= below + (int)hb) {
        s_prefix = pre | ((unsigned long long)tid << shift);
        s_rank = want - below;
        s_bucket = (int)hb;
      }
      __syncthreads();
      mask |= 255ull << shift;
      if (s_bucket == 1 || shift == 0) {
        // one key left in the bucket: it is the threshold
        const unsigned long long pfx = s_prefix;
        for_keys([&](unsigned long long k) {
          if ((k & mask) == pfx) s_thr = k;
        });
        __syncthreads();
        break;
      }
    }
    thr = s_thr;
  }
  // compaction in packed order: accepted rows to off + rank, the rest -1
  int run = 0;
  for (int j0 = 0; j0 < n; j0 += kCapThreads) {
    const int j = j0 + tid;
    int32_t r = -1;
    bool take = false;
    if (j < n) {
      r = src_all[base + j];
      const unsigned long long k = ((unsigned long long)(~float_orderable(gates[r])) << 32) | (uint32_t)r;
      take = C > 0 && k <= thr;
    }
    int tot;
    const int rank = block_exclusive_scan(take ? 1 : 0, scratch, &tot);
    if (j < n) {
      if (take) {
        route_src[off + run + rank] = r;
        route_pos[r] = off + run + rank;
      } else {
        route_pos[r] = -1;
      }
    }
    run += tot;
  }
}

hipError_t launch_capacity(const int32_t* counts_all, const int32_t* offsets_all, const int32_t* src_all,
                           const float* gates, int E, int C, int32_t* counts, int32_t* offsets,
                           int32_t* route_src, int32_t* route_pos, hipStream_t s) {
  if (E <= 0) return hipSuccess;
  hipLaunchKernelGGL(capacity_kernel, dim3(E), dim3(kCapThreads), 0, s, counts_all, offsets_all, src_all, gates, E, C,
                     counts, offsets, route_src, route_pos);
  return hipGetLastError();
}

hipError_t launch_dispatch(const int32_t* ids, int T, int K, int E, int32_t* counts,
                           int32_t* offsets, int32_t* route_src, int32_t* route_pos,
                           void* scratch, const PlanOut* plan, hipStream_t s) {
  const int C = ceil_div(T, kDispatchChunk);
  int32_t* cc = (int32_t*)scratch;
  if (C > 0) hipLaunchKernelGGL(dispatch_count_kernel, dim3(C), dim3(256), 0, s, ids, T, K, E, cc);
  PlanOut P = plan ? *plan : PlanOut{};
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, s, cc, C, E, counts, offsets, P,
                     plan ? 1 : 0);
  if (C > 0)
    hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(C), dim3(256), 0, s, ids, T, K, E, cc, offsets,
                       route_src, route_pos);
  return hipGetLastError();
}

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int E, PlanOut P) {
  __shared__ int s_count[MOE_MAX_EXPERTS];
  __shared__ int s_gstart[MOE_MAX_EXPERTS + 2];
  __shared__ int scratch[32];
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_count[e] = offsets[e + 1] - offsets[e];
  __syncthreads();
  build_plans(s_count, E, P, s_gstart, scratch);
}

hipError_t launch_plan(const int32_t* offsets, const PlanOut* plan, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, offsets, plan->up.E, *plan);
  return hipGetLastError();
}

}  // namespace moe
