// Decode-size batches (at most kDecodeMaxRows rows): the layer in six
// launches, built so that every expert weight byte the batch needs is read
// once from HBM and nothing else is.
//
//  * router_small_kernel: fp32 logits as plain fp32 dot products (bf16 x
//    widened exactly), one wave per (expert, pair of tokens).
//  * dispatch_small_kernel: one workgroup does the histogram, the offsets,
//    the expert-major permutation in (expert, token, slot) order ("M6.1 -
//    Routed Capacity", 0x05A/0x05E) and the list of work items: one item per
//    (touched expert, block of 16 of its rows, chunk of 64 hidden neurons),
//    plus the shared expert's.
//  * expert_decode_kernel: one workgroup per item.  Up projection of the
//    item's 64 neurons for its rows on MFMA 16x16x32 (weights
//    and rows read straight from global memory), ReLU^2 with the rounding
//    points of the NemotronH "Arithmetic" section into LDS, then the down
//    projection of the same 64 neurons reading only the rows of the
//    neuron-major down weights whose neuron is non-zero for some row of the
//    group (the 8 GB Nemotron-3.5-Super write-up, "The engine, step by step",
//    item 4: a zero neuron needs none of its down weights): streamed through
//    registers for items of up to 4 rows, staged through LDS and shared by
//    all rows of larger items.  The item's contribution is written as an
//    fp32 partial row per (group row, chunk).
//  * reduce_chunks_kernel: each row's chunk partials summed in a fixed order,
//    grid-parallel over rows and column blocks.
//  * combine_decode_kernel: per token, the routes in ascending expert id,
//    then the shared expert, one rounding ("NemotronH", "Arithmetic"; no
//    atomics, so the result is deterministic).
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kItemRows = kDecodeItemRows;  // rows of one work item (one 16-row MFMA block)

// ---------------------------------------------------------------------------
// Router logits for small T
// ---------------------------------------------------------------------------
constexpr int kRouterTok = 2;   // tokens per wave
constexpr int kRouterIt = kDecodeMaxWidth / 8 / 64;  // 8-element chunks per lane at the widest row

// One wave per (expert, pair of tokens); every load of the wave is issued
// before the first FMA, so each wave pays one memory latency.
__global__ __launch_bounds__(256) void router_small_kernel(const uint16_t* __restrict__ x, int T, int d,
                                                           const float* __restrict__ w, int E,
                                                           float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t0 = blockIdx.y * kRouterTok;
  if (e >= E) return;
  const int nch = d / 8;  // 8-element chunks of a row
  const float* wr = w + (long)e * d;
  float4 wv[kRouterIt][2];
  uint4 xv[kRouterTok][kRouterIt];
#pragma unroll
  for (int it = 0; it < kRouterIt; ++it) {
    const int c = lane + 64 * it;
    const bool in = c < nch;
    wv[it][0] = in ? *(const float4*)(wr + c * 8) : make_float4(0, 0, 0, 0);
    wv[it][1] = in ? *(const float4*)(wr + c * 8 + 4) : make_float4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < kRouterTok; ++i)
      xv[i][it] = (in && t0 + i < T) ? *(const uint4*)(x + (long)(t0 + i) * d + c * 8) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < kRouterTok; ++i) {
    float acc = 0.0f;
#pragma unroll
    for (int it = 0; it < kRouterIt; ++it) {
      const float wf[8] = {wv[it][0].x, wv[it][0].y, wv[it][0].z, wv[it][0].w,
                           wv[it][1].x, wv[it][1].y, wv[it][1].z, wv[it][1].w};
      const uint32_t u[4] = {xv[i][it].x, xv[i][it].y, xv[i][it].z, xv[i][it].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc = fmaf(bf16_to_f32(u[q] & 0xffffu), wf[2 * q], acc);
        acc = fmaf(bf16_to_f32(u[q] >> 16), wf[2 * q + 1], acc);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0 && t0 + i < T) logits[(long)(t0 + i) * E + e] = acc;
  }
}

hipError_t launch_router_small(const uint16_t* x, int T, int d, const float* w, int E, float* logits,
                               hipStream_t s) {
  dim3 grid(ceil_div(E, 4), ceil_div(T, kRouterTok));
  hipLaunchKernelGGL(router_small_kernel, grid, dim3(256), 0, s, x, T, d, w, E, logits);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dispatch and work list in one workgroup
// ---------------------------------------------------------------------------
// Exclusive scan over the workgroup (blockDim.x <= 1024); *total = the sum.
__device__ int wg_exclusive_scan(int v, int* scratch /*[33]*/, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = (blockDim.x + 63) >> 6;
  int xs = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(xs, off, 64);
    if (lane >= off) xs += y;
  }
  if (lane == 63) scratch[wave] = xs;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      const int q = scratch[w];
      scratch[w] = run;
      run += q;
    }
    scratch[32] = run;
  }
  __syncthreads();
  const int res = scratch[wave] + xs - v;
  *total = scratch[32];
  __syncthreads();
  return res;
}

// Work item (group, 16-row block, 64-neuron chunk) packed in one int32.
__device__ __forceinline__ int decode_item(int g, int rb, int c) { return (g << 20) | (rb << 12) | c; }
// The items of one group: chunk-major, the row blocks of a chunk adjacent so
// they run together and share the chunk's weights in L2.
__device__ __forceinline__ void write_items(int32_t* out, int g, int nrb, int nc) {
  for (int c = 0; c < nc; ++c)
    for (int rb = 0; rb < nrb; ++rb) out[c * nrb + rb] = decode_item(g, rb, c);
}

// The dispatch and the work list, one workgroup of 1024 threads (16 waves).
// The routes are cut into 16 consecutive segments, one per wave:
//  1. per-wave expert histograms (LDS atomics: counts do not depend on order);
//  2. per expert (one thread each): its count, the exclusive offset of every
//     wave's share inside the expert's rows, and the exclusive scan over
//     experts (the offsets);
//  3. each wave walks its segment 64 routes at a time; a route's rank among
//     the lanes of its chunk with the same expert comes from ballots over the
//     expert id's bits, so the packed order is (expert, route index) as in
//     "M6.1 - Routed Capacity", 0x05A / 0x05E;
//  4. the work items: the shared group's first, then the experts' in
//     descending order of their counts, written by all threads (each finds
//     its expert by a binary search over the item offsets of that order).
constexpr int kDispWaves = 16;

__global__ __launch_bounds__(1024) void dispatch_small_kernel(const int32_t* __restrict__ ids, int T, int R,
                                                              int E, int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ route_src,
                                                              int32_t* __restrict__ route_pos,
                                                              int ncr, int ncs,
                                                              int32_t* __restrict__ items,
                                                              int32_t* __restrict__ n_items) {
  __shared__ int s_ids[kDecodeMaxRoutes];
  __shared__ int s_h[kDispWaves * MOE_MAX_EXPERTS];  // [wave][expert]
  __shared__ int s_off[MOE_MAX_EXPERTS], s_cnt[MOE_MAX_EXPERTS], s_ioff[MOE_MAX_EXPERTS + 1];
  __shared__ int scratch[33];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int r = tid; r < R; r += blockDim.x) s_ids[r] = ids[r];
  for (int q = tid; q < kDispWaves * E; q += blockDim.x) s_h[q] = 0;
  __syncthreads();
  const int seg = ceil_div(R, kDispWaves);
  const int r_lo = min(R, wave * seg), r_hi = min(R, r_lo + seg);
  int* h = s_h + wave * E;
  for (int r = r_lo + lane; r < r_hi; r += 64) atomicAdd(&h[s_ids[r]], 1);
  __syncthreads();
  int cnt = 0;
  if (tid < E)
    for (int w = 0; w < kDispWaves; ++w) {
      const int v = s_h[w * E + tid];
      s_h[w * E + tid] = cnt;
      cnt += v;
    }
  int total;
  const int off = wg_exclusive_scan(tid < E ? cnt : 0, scratch, &total);
  if (tid < E) {
    counts[tid] = cnt;
    offsets[tid] = off;
    s_off[tid] = off;
    s_cnt[tid] = cnt;
  }
  if (tid == 0) offsets[E] = total;
  __syncthreads();
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  for (int base = r_lo; base < r_hi; base += 64) {
    const int r = base + lane;
    const bool valid = r < r_hi;
    const int e = valid ? s_ids[r] : 0;
    unsigned long long same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const unsigned long long m = __ballot(valid && bit);
      same &= bit ? m : ~m;
    }
    if (valid) {
      const int rank = __popcll(same & ((1ull << lane) - 1ull));
      const int pos = s_off[e] + h[e] + rank;
      route_src[pos] = r;
      route_pos[r] = pos;
    }
    // every lane has read h[] before the group's last lane advances it
    __builtin_amdgcn_wave_barrier();
    if (valid && (same & ~((2ull << lane) - 1ull)) == 0) h[e] += __popcll(same);
    __builtin_amdgcn_wave_barrier();
  }
  // work items, longest first: the shared group E's (T rows, whose items
  // run longest), then the touched experts' in descending order of their
  // route counts (equal counts: ascending id), each chunk-major with the
  // row blocks of a chunk adjacent.  Workgroups start in item order, so the
  // long items do not form the launch's tail.
  const int nrb_s = ceil_div(T, kItemRows);
  const int n_s = ncs ? nrb_s * ncs : 0;
  int rank = 0;  // position of expert tid in that order
  if (tid < E)
    for (int e = 0; e < E; ++e) {
      const int c2 = s_cnt[e];
      rank += (c2 > cnt || (c2 == cnt && e < tid)) ? 1 : 0;
    }
  __syncthreads();
  if (tid < E) s_h[rank] = tid;  // s_h reused: expert of each rank
  __syncthreads();
  const int e_r = tid < E ? s_h[tid] : 0;
  int itot;
  const int ioff = wg_exclusive_scan(tid < E ? ceil_div(s_cnt[e_r], kItemRows) * ncr : 0, scratch, &itot);
  if (tid < E) s_ioff[tid] = ioff;
  if (tid == 0) s_ioff[E] = itot;
  __syncthreads();
  for (int q = tid; q < n_s; q += blockDim.x) items[q] = decode_item(E, q % nrb_s, q / nrb_s);
  for (int q = tid; q < itot; q += blockDim.x) {
    int lo = 0, hi = E - 1;  // the largest rank with s_ioff[rank] <= q owns item q
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_ioff[mid] <= q)
        lo = mid;
      else
        hi = mid - 1;
    }
    const int e = s_h[lo];
    const int nrb_e = ceil_div(s_cnt[e], kItemRows), l = q - s_ioff[lo];
    items[n_s + q] = decode_item(e, l % nrb_e, l / nrb_e);
  }
  if (tid == 0) *n_items = n_s + itot;
}

hipError_t launch_dispatch_small(const int32_t* ids, int T, int K, int E, int32_t* counts,
                                 int32_t* offsets, int32_t* route_src, int32_t* route_pos, int ncr,
                                 int ncs, int32_t* items, int32_t* n_items, hipStream_t s) {
  hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(1024), 0, s, ids, T, T * K, E, counts, offsets,
                     route_src, route_pos, ncr, ncs, items, n_items);
  return hipGetLastError();
}

// Work list of the staged expert call from existing offsets (no shared group).
__global__ __launch_bounds__(1024) void decode_items_kernel(const int32_t* __restrict__ offsets, int E,
                                                            int ncr, int32_t* __restrict__ items,
                                                            int32_t* __restrict__ n_items) {
  __shared__ int scratch[33];
  int tot = 0;
  for (int base = 0; base < E; base += blockDim.x) {
    const int e = base + threadIdx.x;
    const int cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
    const int nrb = ceil_div(cnt, kItemRows);
    int seg;
    const int o = wg_exclusive_scan(nrb * ncr, scratch, &seg);
    if (e < E) write_items(items + tot + o, e, nrb, ncr);
    tot += seg;
  }
  if (threadIdx.x == 0) *n_items = tot;
}

hipError_t launch_decode_items(const int32_t* offsets, int E, int ncr, int32_t* items,
                               int32_t* n_items, hipStream_t s) {
  hipLaunchKernelGGL(decode_items_kernel, dim3(1), dim3(1024), 0, s, offsets, E, ncr, items, n_items);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused up + ReLU^2 + zero-skipping down, one (group, 64-neuron chunk) item
// per workgroup
// ---------------------------------------------------------------------------
constexpr int kChunkN = kDecodeChunk;
constexpr int kUnroll = 8;    // k32 steps of loads in flight per wave

// Weight formats of the expert matrices: bf16, FP8 E4M3 codes, MXFP4 codes.
constexpr int kWBf16 = 0, kWFp8 = 1, kWFp4 = 2;
// Bytes of n weights in format WF.
template <int WF>
__host__ __device__ constexpr long wbytes(long n) {
  return WF == kWFp4 ? n / 2 : WF == kWFp8 ? n : 2 * n;
}

struct GroupView {
  int M;                      // rows of the item (<= kItemRows)
  long prow;                  // partial row of the item's first row
  const uint16_t* x;          // input rows
  long ldx;
  const int32_t* src;         // item row -> route (NULL: x row xrow0 + row)
  long xrow0;
  int K;
  int Kd;                     // input width
  int F;                      // hidden width
  const char* w_up;           // [F][Kd], packed (bf16, or FP8 codes)
  const char* w_dn;           // [F][Nd] neuron-major, packed
  const float* s_up;          // FP8: [F] up scales
  const float* s_dn;          // FP8: [Nd] down scales
  const uint8_t* e_up;        // MXFP4: [Kd / 32][F] up scales
  const uint8_t* e_dn;        // MXFP4: [F / 32][Nd] down scales
  int Nd;                     // output width
  float* part;                // [*][nc][Nd]
  int nc;
};

// The item's view of group g, rows [rb * kItemRows, rb * kItemRows + kItemRows).
// A routed group's rows are packed rows o .. o + Mg - 1, whose routes are
// src[o ..] (src: the dispatch's route order in global memory or LDS).
template <int WF>
__device__ __forceinline__ GroupView decode_group(const DecodeArgs& a, int g, int rb, int o, int Mg,
                                                  const int32_t* src) {
  constexpr bool W8 = WF == kWFp8, W4 = WF == kWFp4;
  GroupView v;
  const int r0 = rb * kItemRows;
  if (g < a.E) {
    v.prow = o + r0;
    v.x = a.x;
    v.ldx = a.ldx;
    v.src = src ? src + o + r0 : nullptr;
    v.xrow0 = o + r0;
    v.K = a.K;
    v.Kd = a.d_e;
    v.F = a.F;
    v.w_up = (const char*)a.w_up + wbytes<WF>((long)g * a.F * a.d_e);
    v.w_dn = (const char*)a.w_dn + wbytes<WF>((long)g * a.F * a.d_e);
    v.s_up = W8 ? a.s_up + (long)g * a.F : nullptr;
    v.s_dn = W8 ? a.s_dn + (long)g * a.d_e : nullptr;
    v.e_up = W4 ? a.e_up + (long)g * a.F * (a.d_e / kMxBlock) : nullptr;
    v.e_dn = W4 ? a.e_dn + (long)g * a.d_e * (a.F / kMxBlock) : nullptr;
    v.Nd = a.d_e;
    v.part = a.part;
    v.nc = a.ncr;
  } else {
    Mg = a.M_s;
    v.prow = r0;
    v.x = a.x_s;
    v.ldx = a.ldx_s;
    v.src = nullptr;
    v.xrow0 = r0;
    v.K = 1;
    v.Kd = a.d_s;
    v.F = a.F_s;
    v.w_up = (const char*)a.w_up_s;
    v.w_dn = (const char*)a.w_dn_s;
    v.s_up = a.s_up_s;
    v.s_dn = a.s_dn_s;
    v.e_up = a.e_up_s;
    v.e_dn = a.e_dn_s;
    v.Nd = a.d_s;
    v.part = a.part_s;
    v.nc = a.ncs;
  }
  v.M = min(kItemRows, Mg - r0);
  return v;
}

constexpr int kColBlock = kPackTile;  // output columns per LDS-staged block: one strip of the packed down weights
constexpr int kRegRows = 4;     // items of at most this many rows stream the down weights through registers
constexpr int kLiveUnroll = 8;  // live neurons in flight per thread on the register path

// Eight consecutive weights of one row as fp32: 16 bytes of bf16 (w) or the
// low 8 bytes of FP8 codes (w.x, w.y).
template <bool W8>
__device__ __forceinline__ void weights8(const uint4& w, float (&f)[8]) {
  if (W8) {
    fp8x8_to_f32(make_uint2(w.x, w.y), f);
  } else {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[2 * q] = bf16_to_f32(u[q] & 0xffffu);
      f[2 * q + 1] = bf16_to_f32(u[q] >> 16);
    }
  }
}
// Eight consecutive weights at p (16 bytes of bf16 or 8 bytes of codes).
template <bool W8>
__device__ __forceinline__ uint4 load8(const char* p) {
  if (W8) {
    const uint2 q = *(const uint2*)p;
    return make_uint4(q.x, q.y, 0, 0);
  }
  return *(const uint4*)p;
}
// FP8: multiply 8 fp32 sums of columns col .. col+7 by their down scales.
template <int WF>
__device__ __forceinline__ void scale8(const GroupView& v, int col, float* acc) {
  if (WF != kWFp8) return;
  const float4 s0 = *(const float4*)(v.s_dn + col), s1 = *(const float4*)(v.s_dn + col + 4);
  acc[0] *= s0.x; acc[1] *= s0.y; acc[2] *= s0.z; acc[3] *= s0.w;
  acc[4] *= s1.x; acc[5] *= s1.y; acc[6] *= s1.z; acc[7] *= s1.w;
}

// Down projection of the live neurons for an item of at most kRegRows rows:
// a thread owns a group of output columns (two groups of 8 for bf16 when
// the width needs them, one group of 16 for FP8 codes: 16 bytes of weights
// per neuron either way) and walks the live neurons kLiveUnroll at a time,
// so every live weight row is read once, with several rows in flight.
template <bool W8, int RR>
__device__ __forceinline__ void down_small(const GroupView& v, int c, int nbase, const uint16_t* s_ht,
                                           const int* s_live, int nlive) {
  static_assert(RR == 1 || RR == 2 || RR == 4, "rows held in registers");
  constexpr long eb = W8 ? 1 : 2;
  constexpr int kCols = W8 ? 16 : 8;   // columns of a group
  constexpr int kGroups = W8 ? 1 : 2;  // groups per thread (widths up to 4096)
  const int tid = threadIdx.x;
  const int ncg = v.Nd / kCols;
  bool has[kGroups];
  int cn[kGroups];
  const char* wb[kGroups];
#pragma unroll
  for (int j = 0; j < kGroups; ++j) {
    const int cg = tid + 256 * j;
    has[j] = cg < ncg;
    // packed neuron-major: column col of neuron f at strip(col) * F + f * width(strip) + col - strip
    const int c0 = (cg * kCols) & ~(kPackTile - 1);
    cn[j] = min(kPackTile, v.Nd - c0);
    wb[j] = v.w_dn + ((long)c0 * v.F + (cg * kCols - c0)) * eb;
  }
  const int M = v.M;
  float acc[kGroups][RR][kCols];
#pragma unroll
  for (int j = 0; j < kGroups; ++j)
#pragma unroll
    for (int r = 0; r < RR; ++r)
#pragma unroll
      for (int q = 0; q < kCols; ++q) acc[j][r][q] = 0.0f;
  for (int i0 = 0; i0 < nlive; i0 += kLiveUnroll) {
    uint4 w[kGroups][kLiveUnroll];
    int fl[kLiveUnroll];
#pragma unroll
    for (int u = 0; u < kLiveUnroll; ++u) {
      const int i = i0 + u;
      fl[u] = i < nlive ? s_live[i] : -1;
      const long f = nbase + (fl[u] < 0 ? 0 : fl[u]);
#pragma unroll
      for (int j = 0; j < kGroups; ++j)
        w[j][u] = (fl[u] >= 0 && has[j]) ? *(const uint4*)(wb[j] + f * cn[j] * eb) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kLiveUnroll; ++u) {
      if (fl[u] < 0) break;
      // h of this neuron for rows 0..RR-1 (rows >= M hold zeros)
      const uint2 hv2 = *(const uint2*)(s_ht + fl[u] * kItemRows);
      const float hv[4] = {bf16_to_f32(hv2.x & 0xffffu), bf16_to_f32(hv2.x >> 16),
                           bf16_to_f32(hv2.y & 0xffffu), bf16_to_f32(hv2.y >> 16)};
#pragma unroll
      for (int j = 0; j < kGroups; ++j) {
        float f[kCols];
        if constexpr (W8) {
          float lo[8], hi[8];
          fp8x8_to_f32(make_uint2(w[j][u].x, w[j][u].y), lo);
          fp8x8_to_f32(make_uint2(w[j][u].z, w[j][u].w), hi);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            f[q] = lo[q];
            f[8 + q] = hi[q];
          }
        } else {
          float b8[8];
          weights8<false>(w[j][u], b8);
#pragma unroll
          for (int q = 0; q < 8; ++q) f[q] = b8[q];
        }
#pragma unroll
        for (int q = 0; q < kCols; ++q)
#pragma unroll
          for (int r = 0; r < RR; ++r) acc[j][r][q] = fmaf(hv[r], f[q], acc[j][r][q]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RR; ++r) {
    if (r >= M) break;
    float* prow = v.part + ((v.prow + r) * v.nc + c) * (long)v.Nd;
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
      if (!has[j]) continue;
      const int col = (tid + 256 * j) * kCols;
#pragma unroll
      for (int q = 0; q < kCols; q += 8) {
        scale8<W8 ? kWFp8 : kWBf16>(v, col + q, &acc[j][r][q]);
        *(float4*)(prow + col + q) = make_float4(acc[j][r][q], acc[j][r][q + 1], acc[j][r][q + 2], acc[j][r][q + 3]);
        *(float4*)(prow + col + q + 4) =
            make_float4(acc[j][r][q + 4], acc[j][r][q + 5], acc[j][r][q + 6], acc[j][r][q + 7]);
      }
    }
  }
}

// Down projection of the live neurons for items of kRegRows+1 .. kItemRows
// rows: the live weight rows are staged through LDS one block of columns at a
// time (read from memory once: 512 bytes a row, one strip of 256 bf16
// columns or two strips of FP8 codes) and every row of the item reuses them.
// Thread layout per block: 32 column groups x 8 row lanes of 2 rows.
template <bool W8>
__device__ __forceinline__ void down_large(const GroupView& v, int c, int nbase, const uint16_t* s_ht,
                                           const int* s_live, int nlive, char* s_w) {
  constexpr int eb = W8 ? 1 : 2;
  constexpr int kBlk = W8 ? 2 * kColBlock : kColBlock;  // columns of a staged block
  constexpr int kRowB = kBlk * eb;                       // bytes of a staged row
  constexpr int kPieces = kRowB / 16;                    // 16-byte pieces of a staged row
  constexpr int kCols = kBlk / 32;                       // columns of a thread's group
  constexpr int kPer = kChunkN * kPieces / 256;          // pieces a thread stages per block (at most)
  const int tid = threadIdx.x;
  const int cgl = tid & 31, r0 = (tid >> 5) * 2;
  const int M = v.M;
  const int nblk = ceil_div(v.Nd, kBlk);
  const int npieces = nlive * kPieces;
  // the staged pieces of a block: idx = tid + 256 u -> (live row i, piece
  // q); a piece lies in one strip of the packed layout (row-major [F][cn]
  // from column sc0).  All of a block's loads are issued together, and the
  // next block's while the current one is computed.
  uint4 wbuf[kPer];
  auto load_block = [&](int cb) {
    const int col0 = cb * kBlk;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int idx = tid + 256 * u;
      wbuf[u] = make_uint4(0, 0, 0, 0);
      if (idx < npieces) {
        const int i = idx / kPieces, q = idx % kPieces;
        const int pc = col0 + q * (16 / eb);  // the piece's first column
        const int sc0 = pc & ~(kPackTile - 1);
        const int cn = min(kPackTile, v.Nd - sc0);
        if (pc < v.Nd)
          wbuf[u] = *(const uint4*)(v.w_dn + ((long)sc0 * v.F + (long)(nbase + s_live[i]) * cn + (pc - sc0)) * eb);
      }
    }
  };
  load_block(0);
  for (int cb = 0; cb < nblk; ++cb) {
    const int col0 = cb * kBlk;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int idx = tid + 256 * u;
      if (idx < npieces) *(uint4*)(s_w + (idx / kPieces) * kRowB + (idx % kPieces) * 16) = wbuf[u];
    }
    __syncthreads();
    if (cb + 1 < nblk) load_block(cb + 1);
    const int col = col0 + cgl * kCols;
    float acc[2][kCols];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < kCols; ++q) acc[j][q] = 0.0f;
    if (r0 < M) {
      for (int i = 0; i < nlive; ++i) {
        const uint4 wv = *(const uint4*)(s_w + i * kRowB + cgl * 16);
        const uint32_t hu = *(const uint32_t*)(s_ht + s_live[i] * kItemRows + r0);
        const float h0 = bf16_to_f32(hu & 0xffffu), h1 = bf16_to_f32(hu >> 16);
        float wf[kCols];
        if constexpr (W8) {
          float lo[8], hi[8];
          fp8x8_to_f32(make_uint2(wv.x, wv.y), lo);
          fp8x8_to_f32(make_uint2(wv.z, wv.w), hi);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            wf[q] = lo[q];
            wf[q + 8] = hi[q];
          }
        } else {
          float b8[8];
          weights8<false>(wv, b8);
#pragma unroll
          for (int q = 0; q < 8; ++q) wf[q] = b8[q];
        }
#pragma unroll
        for (int q = 0; q < kCols; ++q) {
          acc[0][q] = fmaf(h0, wf[q], acc[0][q]);
          acc[1][q] = fmaf(h1, wf[q], acc[1][q]);
        }
      }
    }
    if (col < v.Nd) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (r0 + j >= M) break;
        float* prow = v.part + ((v.prow + r0 + j) * v.nc + c) * (long)v.Nd + col;
#pragma unroll
        for (int q = 0; q < kCols; q += 8) {
          scale8<W8 ? kWFp8 : kWBf16>(v, col + q, &acc[j][q]);
          *(float4*)(prow + q) = make_float4(acc[j][q], acc[j][q + 1], acc[j][q + 2], acc[j][q + 3]);
          *(float4*)(prow + q + 4) = make_float4(acc[j][q + 4], acc[j][q + 5], acc[j][q + 6], acc[j][q + 7]);
        }
      }
    }
    __syncthreads();
  }
}

// MXFP4 down projection of the live neurons, items of at most kRegRows
// rows: a thread owns 16 output columns (8 bytes of codes per neuron; widths
// up to 4096).  The item's 64 neurons lie in two scale blocks, whose scales
// for the thread's columns are read once; the live list is ascending, so its
// first nlo neurons are block 0's and the walk takes each block with its
// scales in registers.  Each code is widened to fp32 and multiplied by its
// column's scale (exact) before the FMAs.
template <int RR>
__device__ __forceinline__ void down_small_fp4(const GroupView& v, int c, int nbase, const uint16_t* s_ht,
                                               const int* s_live, int nlive, int nlo) {
  static_assert(RR == 1 || RR == 2 || RR == 4, "rows held in registers");
  constexpr int kCols = 16;
  const int tid = threadIdx.x;
  const bool has = tid < v.Nd / kCols;
  const int fg0 = nbase / kMxBlock, nfg = v.F / kMxBlock;
  const int c0 = (tid * kCols) & ~(kPackTile - 1);
  const int cn = min(kPackTile, v.Nd - c0);
  const char* wb = v.w_dn + ((long)c0 * v.F + (tid * kCols - c0)) / 2;
  const int M = v.M;
  float acc[RR][kCols];
#pragma unroll
  for (int r = 0; r < RR; ++r)
#pragma unroll
    for (int q = 0; q < kCols; ++q) acc[r][q] = 0.0f;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int fg = fg0 + blk;
    const uint4 e = (has && fg < nfg) ? *(const uint4*)(v.e_dn + (long)fg * v.Nd + tid * kCols) : make_uint4(0, 0, 0, 0);
    const uint32_t ew[4] = {e.x, e.y, e.z, e.w};
    float sc[kCols];
#pragma unroll
    for (int q = 0; q < kCols; ++q) sc[q] = e8m0_to_f32((ew[q >> 2] >> (8 * (q & 3))) & 0xffu);
    const int lo = blk ? nlo : 0, hi = blk ? nlive : nlo;
    for (int i0 = lo; i0 < hi; i0 += kLiveUnroll) {
      uint2 w[kLiveUnroll];
      int fl[kLiveUnroll];
#pragma unroll
      for (int u = 0; u < kLiveUnroll; ++u) {
        const int i = i0 + u;
        fl[u] = i < hi ? s_live[i] : -1;
        const long f = nbase + (fl[u] < 0 ? 0 : fl[u]);
        w[u] = (fl[u] >= 0 && has) ? *(const uint2*)(wb + f * cn / 2) : make_uint2(0, 0);
      }
#pragma unroll
      for (int u = 0; u < kLiveUnroll; ++u) {
        if (fl[u] < 0) break;
        const uint2 hv2 = *(const uint2*)(s_ht + fl[u] * kItemRows);
        const float hv[4] = {bf16_to_f32(hv2.x & 0xffffu), bf16_to_f32(hv2.x >> 16),
                             bf16_to_f32(hv2.y & 0xffffu), bf16_to_f32(hv2.y >> 16)};
        float f[kCols];
        fp4x8_to_f32(w[u].x, *(float(*)[8])&f[0]);
        fp4x8_to_f32(w[u].y, *(float(*)[8])&f[8]);
#pragma unroll
        for (int q = 0; q < kCols; ++q) {
          const float wq = f[q] * sc[q];
#pragma unroll
          for (int r = 0; r < RR; ++r) acc[r][q] = fmaf(hv[r], wq, acc[r][q]);
        }
      }
    }
  }
  if (!has) return;
#pragma unroll
  for (int r = 0; r < RR; ++r) {
    if (r >= M) break;
    float* prow = v.part + ((v.prow + r) * v.nc + c) * (long)v.Nd + tid * kCols;
#pragma unroll
    for (int q = 0; q < kCols; q += 4) *(float4*)(prow + q) = make_float4(acc[r][q], acc[r][q + 1], acc[r][q + 2], acc[r][q + 3]);
  }
}

// MXFP4 down projection for items of kRegRows+1 .. kItemRows rows: the live
// rows' codes are staged through LDS a block of 512 columns at a time (256
// bytes a row) and every row of the item reuses them; a thread owns 16
// columns (8 bytes of codes) for two rows, with the scales of its columns in
// the item's two scale blocks read once per column block.  The live list is
// ascending, so its first nlo neurons are scale block 0's: the walk takes
// each block with its scales in registers.
__device__ __forceinline__ void down_large_fp4(const GroupView& v, int c, int nbase, const uint16_t* s_ht,
                                               const int* s_live, int nlive, int nlo, char* s_w) {
  constexpr int kBlk = 512;
  constexpr int kRowB = kBlk / 2;
  constexpr int kPieces = kRowB / 16;  // 16-byte pieces of 32 columns
  constexpr int kCols = kBlk / 32;     // columns of a thread
  constexpr int kPer = kChunkN * kPieces / 256;  // pieces a thread stages per block (at most)
  const int tid = threadIdx.x;
  const int cgl = tid & 31, r0 = (tid >> 5) * 2;
  const int M = v.M;
  const int fg0 = nbase / kMxBlock, nfg = v.F / kMxBlock;
  const int nblk = ceil_div(v.Nd, kBlk);
  const int npieces = nlive * kPieces;
  // as down_large: a block's loads issued together, the next block's while
  // the current one is computed
  uint4 wbuf[kPer];
  auto load_block = [&](int cb) {
    const int col0 = cb * kBlk;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int idx = tid + 256 * u;
      wbuf[u] = make_uint4(0, 0, 0, 0);
      if (idx < npieces) {
        const int i = idx / kPieces, q = idx % kPieces;
        const int pc = col0 + q * 32;
        const int sc0 = pc & ~(kPackTile - 1);
        const int cn = min(kPackTile, v.Nd - sc0);
        if (pc < v.Nd)
          wbuf[u] = *(const uint4*)(v.w_dn + ((long)sc0 * v.F + (long)(nbase + s_live[i]) * cn + (pc - sc0)) / 2);
      }
    }
  };
  load_block(0);
  for (int cb = 0; cb < nblk; ++cb) {
    const int col0 = cb * kBlk;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int idx = tid + 256 * u;
      if (idx < npieces) *(uint4*)(s_w + (idx / kPieces) * kRowB + (idx % kPieces) * 16) = wbuf[u];
    }
    __syncthreads();
    if (cb + 1 < nblk) load_block(cb + 1);
    const int col = col0 + cgl * kCols;
    float sc[2][kCols];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int fg = fg0 + b;
      const uint4 e = (col < v.Nd && fg < nfg) ? *(const uint4*)(v.e_dn + (long)fg * v.Nd + col) : make_uint4(0, 0, 0, 0);
      const uint32_t ew[4] = {e.x, e.y, e.z, e.w};
#pragma unroll
      for (int q = 0; q < kCols; ++q) sc[b][q] = e8m0_to_f32((ew[q >> 2] >> (8 * (q & 3))) & 0xffu);
    }
    float acc[2][kCols];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < kCols; ++q) acc[j][q] = 0.0f;
    if (r0 < M) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int lo = b ? nlo : 0, hi = b ? nlive : nlo;
        for (int i = lo; i < hi; ++i) {
          const uint2 wv = *(const uint2*)(s_w + i * kRowB + cgl * 8);
          const uint32_t hu = *(const uint32_t*)(s_ht + s_live[i] * kItemRows + r0);
          const float h0 = bf16_to_f32(hu & 0xffffu), h1 = bf16_to_f32(hu >> 16);
          float f[kCols];
          fp4x8_to_f32(wv.x, *(float(*)[8])&f[0]);
          fp4x8_to_f32(wv.y, *(float(*)[8])&f[8]);
#pragma unroll
          for (int q = 0; q < kCols; ++q) {
            const float wq = f[q] * sc[b][q];
            acc[0][q] = fmaf(h0, wq, acc[0][q]);
            acc[1][q] = fmaf(h1, wq, acc[1][q]);
          }
        }
      }
    }
    if (col < v.Nd) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (r0 + j >= M) break;
        float* prow = v.part + ((v.prow + r0 + j) * v.nc + c) * (long)v.Nd + col;
#pragma unroll
        for (int q = 0; q < kCols; q += 4)
          *(float4*)(prow + q) = make_float4(acc[j][q], acc[j][q + 1], acc[j][q + 2], acc[j][q + 3]);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Small batches (T <= kFusedRows, E <= kFusedExperts): the shared group's
// items take the first workgroups, which need no routing; every other
// workgroup routes the T rows from the router logits and builds the dispatch
// in LDS, the same computation as the route and dispatch kernels (the router
// routine is shared; expert counts, offsets by an exclusive scan, each
// expert's routes in route order, work items of the touched experts in
// ascending id, a chunk per item).  Every routing workgroup reaches the same
// dispatch, so it finds its own item without a round trip through memory;
// the first of them also stores ids, weights, counts, offsets and the route
// maps for the combine.  With T <= 16 rows a group is a single row block.
// ---------------------------------------------------------------------------
constexpr int kFusedRoutes = kFusedRows * MOE_MAX_TOPK;
static_assert(kFusedRows <= kItemRows, "a fused batch's group must fit one row block");
static_assert(kFusedRows % 4 == 0 && kFusedExperts <= 128, "four waves route, two scores per lane");

struct FusedDispatch {
  int ids[kFusedRoutes];    // route t*K+k -> expert
  int src[kFusedRoutes];    // packed row -> route
  int off[kFusedExperts];   // expert -> first packed row
  int cnt[kFusedExperts];   // expert -> rows
  int scan[33];
  int pick;
};

// The workgroup's item (g, c), g = E for the shared group, routing and
// dispatching the batch when it is not a shared item.  Returns false when
// the workgroup has no item.  s_route:
// LDS scratch of 4 x 2 x 128 floats.
__device__ bool fused_item(const DecodeArgs& a, float* s_route, FusedDispatch& fd, int* g_out, int* c_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, K = a.K, E = a.E, R = T * K;
  // the shared group's items come first: they need no routing, so their
  // weights stream while the other workgroups route
  const int ns = a.M_s > 0 ? a.ncs : 0;
  if ((int)blockIdx.x < ns) {
    *g_out = E;
    *c_out = blockIdx.x;
    return true;
  }
  const bool writer = (int)blockIdx.x == ns;  // stores the dispatch the combine reads
  float* s_sig = s_route + wave * 256;
  float* s_cor = s_sig + 128;
  for (int j = 0; j < (T + 3) / 4; ++j) {  // T is uniform: every wave runs every pass
    const int t = wave + 4 * j;
    const bool valid = t < T;
    int id;
    float w;
    route_row<2>(a.logits, 1, 0, a.bias, t, valid, E, K, a.n_group, a.topk_group, a.norm, a.rsf, s_sig, s_cor,
                 lane, &id, &w);
    if (valid && lane < K) {
      fd.ids[t * K + lane] = id;
      if (writer) {
        a.ids_out[t * K + lane] = id;
        a.wts_out[t * K + lane] = w;
      }
    }
    __syncthreads();  // the wave's score rows are rewritten by its next row
  }
  // expert tid: its route count, first packed row, and routes in route order
  int cnt = 0;
  if (tid < E)
    for (int r = 0; r < R; ++r) cnt += fd.ids[r] == tid;
  int total;
  const int off = wg_exclusive_scan(tid < E ? cnt : 0, fd.scan, &total);
  if (tid < E) {
    fd.off[tid] = off;
    fd.cnt[tid] = cnt;
    if (writer) {
      a.counts_out[tid] = cnt;
      a.offsets_out[tid] = off;
      if (tid == E - 1) a.offsets_out[E] = off + cnt;
    }
    int n = 0;
    for (int r = 0; r < R; ++r)
      if (fd.ids[r] == tid) {
        fd.src[off + n] = r;
        if (writer) {
          a.rpos_out[r] = off + n;
          a.src_out[off + n] = r;
        }
        ++n;
      }
  }
  // items after the shared group's: a.ncr chunks of each touched expert in
  // ascending id
  int ntouch;
  const bool touched = tid < E && cnt > 0;
  const int rank = wg_exclusive_scan(touched ? 1 : 0, fd.scan, &ntouch);
  const int b = blockIdx.x - ns, nr = ntouch * a.ncr;
  if (touched && b < nr && rank == b / a.ncr) fd.pick = tid;
  __syncthreads();
  if (b < nr) {
    *g_out = fd.pick;
    *c_out = b - (b / a.ncr) * a.ncr;
    return true;
  }
  return false;
}

template <int WF, bool FUSED>
__global__ __launch_bounds__(256, 3) void expert_decode_kernel(DecodeArgs a) {
  constexpr bool W8 = WF == kWFp8, W4 = WF == kWFp4;
  // h of the item's neurons, transposed: s_ht[neuron][row], rows >= M zero
  __shared__ __align__(16) uint16_t s_ht[kChunkN * kItemRows];
  __shared__ __align__(16) char s_w[kChunkN * kColBlock * 2];
  __shared__ int s_live[kChunkN];
  __shared__ int s_nlive, s_nlo;
  int g, rb, c, o = 0, Mg = 0;
  const int32_t* src = nullptr;
  if constexpr (FUSED) {
    __shared__ FusedDispatch fd;
    if (!fused_item(a, (float*)s_w, fd, &g, &c)) return;
    rb = 0;
    if (g < a.E) {
      o = fd.off[g];
      Mg = fd.cnt[g];
      src = fd.src;
    }
  } else {
    if ((int)blockIdx.x >= *a.n_items) return;
    const int item = a.items[blockIdx.x];
    g = item >> 20;
    rb = (item >> 12) & 0xff;
    c = item & 0xfff;
    if (g < a.E) {
      o = a.offsets[g];
      Mg = a.offsets[g + 1] - o;
      src = a.route_src;
    }
  }
  const GroupView v = decode_group<WF>(a, g, rb, o, Mg, src);
  const int M = v.M;
  if (M <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nbase = c * kChunkN;

  // ---- up projection of 16 rows: wave owns neurons nbase + 16 wave .. +15 ----
  const int n_l = nbase + wave * 16 + (lane & 15);
  const int g16 = lane >> 4;  // the lane's k group
  // packed [out][in]: the neuron's 256-row tile, k step k0 is a [rn][32] block
  // (the last, ragged step [rn][Kd - k0])
  const int nc = min(n_l, v.F - 1), r0 = nc & ~(kPackTile - 1), rn = min(kPackTile, v.F - r0);
  const char* wtile = v.w_up + wbytes<WF>((long)r0 * v.Kd);
  const int nrow = nc - r0;
  const int rr = min(lane & 15, M - 1);
  const long xr = v.src ? (long)(v.src[rr] / v.K) : v.xrow0 + rr;
  const uint16_t* xrow = v.x + xr * v.ldx;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (WF == kWBf16) {
    // k32 steps: lane group g takes k = 8g .. 8g+7 of the step (16 bytes)
    const int ksub = g16 * 8;
    for (int k0 = 0; k0 < v.Kd; k0 += 32 * kUnroll) {
      uint4 bw[kUnroll], ax[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int k = k0 + u * 32;
        const bool kin = k + ksub < v.Kd;
        const int kw = min(kPackStep, v.Kd - k);
        bw[u] = kin ? *(const uint4*)(wtile + ((long)k * rn + nrow * kw + ksub) * 2) : make_uint4(0, 0, 0, 0);
        ax[u] = kin ? *(const uint4*)(xrow + k + ksub) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ax[u]),
                                                      __builtin_bit_cast(bf16x8_t, bw[u]), acc, 0, 0, 0);
    }
  } else if constexpr (W8) {
    // FP8 codes, k64 steps: lane group g reads 16 codes, k = 16g .. 16g+15
    // of the step (half g & 1 of the step's k32 block g >> 1), and the x
    // values at the same k; the first 8 go to one MFMA, the last 8 to a
    // second one.  Every k of the step is used once, so the sum is the dot
    // product (Kd is a multiple of 16: a group is all in or all out).
    const int kg = g16 * 16;
    for (int k0 = 0; k0 < v.Kd; k0 += 64 * kUnroll) {
      uint4 bw[kUnroll], a0[kUnroll], a1[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int k = k0 + u * 64 + kg;  // the lane's first k
        const bool kin = k < v.Kd;
        const int kb = k & ~(kPackStep - 1);  // its k32 block
        const int kw = min(kPackStep, v.Kd - kb);
        bw[u] = kin ? *(const uint4*)(wtile + (long)kb * rn + nrow * kw + (k - kb)) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int k = k0 + u * 64 + kg;
        const bool kin = k < v.Kd;
        a0[u] = kin ? *(const uint4*)(xrow + k) : make_uint4(0, 0, 0, 0);
        a1[u] = kin ? *(const uint4*)(xrow + k + 8) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint4 b0 = fp8x8_to_bf16x8(make_uint2(bw[u].x, bw[u].y));
        const uint4 b1 = fp8x8_to_bf16x8(make_uint2(bw[u].z, bw[u].w));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0[u]),
                                                      __builtin_bit_cast(bf16x8_t, b0), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1[u]),
                                                      __builtin_bit_cast(bf16x8_t, b1), acc, 0, 0, 0);
      }
    }
  } else {
    // MXFP4 codes, k128 steps: lane group g reads the 16 bytes (32 codes, one
    // scale block) of the step's k32 block g, k = 32g .. 32g+31, and the x
    // values at the same k; its four 8-code pieces, widened with the block's
    // scale (exact), go to four MFMAs.  Every k of the step is used once, so
    // the sum is the dot product (Kd is a multiple of 32: a block is all in
    // or all out).
    constexpr int kU4 = 4;
    const int kg = g16 * 32;
    for (int k0 = 0; k0 < v.Kd; k0 += 128 * kU4) {
      uint4 bw[kU4], ax[kU4][4];
      float sc[kU4];
#pragma unroll
      for (int u = 0; u < kU4; ++u) {
        const int k = k0 + u * 128 + kg;
        const bool kin = k < v.Kd;
        bw[u] = kin ? *(const uint4*)(wtile + ((long)k * rn + nrow * 32) / 2) : make_uint4(0, 0, 0, 0);
        sc[u] = kin ? e8m0_to_f32(v.e_up[(long)(k / kMxBlock) * v.F + nc]) : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kU4; ++u) {
        const int k = k0 + u * 128 + kg;
        const bool kin = k < v.Kd;
#pragma unroll
        for (int i = 0; i < 4; ++i) ax[u][i] = kin ? *(const uint4*)(xrow + k + 8 * i) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kU4; ++u) {
        const uint32_t wq[4] = {bw[u].x, bw[u].y, bw[u].z, bw[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ax[u][i]),
                                                        __builtin_bit_cast(bf16x8_t, fp4x8_to_bf16x8(wq[i], sc[u])),
                                                        acc, 0, 0, 0);
      }
    }
  }
  // D layout of the 16x16 MFMA: lane l, element i holds row 4*(l/16) + i,
  // column l%16.  FP8: the neuron's scale times the fp32 sum.  ReLU^2 with
  // bf16 rounding before and after the square; rows past M are stored as
  // zeros.
  const float su = (W8 && n_l < v.F) ? v.s_up[n_l] : 1.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * (lane >> 4) + i;
    float h = 0.0f;
    if (row < M && n_l < v.F) {
      const float u = W8 ? acc[i] * su : acc[i];
      const float r = fmaxf(bf16_round(u), 0.0f);
      h = r * r;
    }
    s_ht[(wave * 16 + (lane & 15)) * kItemRows + row] = (uint16_t)f32_to_bf16(h);
  }
  __syncthreads();

  // ---- live neurons of the chunk: non-zero for at least one row ----
  if (wave == 0) {
    const int n = nbase + lane;
    bool live = false;
    long zeros = 0;
    if (n < v.F)
      for (int r = 0; r < M; ++r) {
        const bool nz = (s_ht[lane * kItemRows + r] & 0x7fffu) != 0;
        live |= nz;
        zeros += nz ? 0 : 1;
      }
    const unsigned long long b = __ballot(live);
    const unsigned long long below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    if (live) s_live[__popcll(b & below)] = lane;
    if (lane == 0) {
      s_nlive = __popcll(b);
      s_nlo = __popcll(b & 0xffffffffull);  // live neurons of the chunk's first 32
    }
    if (a.zero_count) {
      unsigned long long zs = (unsigned long long)zeros;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) zs += __shfl_xor(zs, off, 64);
      const int valid = min(kChunkN, v.F - nbase);
      if (lane == 0) {
        const int slot = g < a.E ? 0 : 2;
        atomicAdd(&a.zero_count[slot], zs);
        atomicAdd(&a.zero_count[slot + 1], (unsigned long long)(valid - __popcll(b)));
      }
    }
  }
  __syncthreads();
  const int nlive = s_nlive;
  // items of at most kRegRows rows keep 1, 2 or 4 rows in registers
  if constexpr (W4) {
    const int nlo = s_nlo;
    if (M == 1)
      down_small_fp4<1>(v, c, nbase, s_ht, s_live, nlive, nlo);
    else if (M == 2)
      down_small_fp4<2>(v, c, nbase, s_ht, s_live, nlive, nlo);
    else if (M <= kRegRows)
      down_small_fp4<4>(v, c, nbase, s_ht, s_live, nlive, nlo);
    else
      down_large_fp4(v, c, nbase, s_ht, s_live, nlive, nlo, s_w);
  } else if (M == 1) {
    down_small<W8, 1>(v, c, nbase, s_ht, s_live, nlive);
  } else if (M == 2) {
    down_small<W8, 2>(v, c, nbase, s_ht, s_live, nlive);
  } else if (M <= kRegRows) {
    down_small<W8, 4>(v, c, nbase, s_ht, s_live, nlive);
  } else {
    down_large<W8>(v, c, nbase, s_ht, s_live, nlive, s_w);
  }
}

hipError_t launch_expert_decode(const DecodeArgs& a, int max_items, hipStream_t s) {
  if (max_items <= 0) return hipSuccess;
  if (a.w8 && a.w4) return hipErrorInvalidValue;
  if (a.w4 && (a.d_e % kMxBlock || a.F % kMxBlock || (a.M_s && (a.d_s % kMxBlock || a.F_s % kMxBlock))))
    return hipErrorInvalidValue;
  if (a.fused && (a.T < 1 || a.T > kFusedRows || a.E > kFusedExperts || a.K > MOE_MAX_TOPK))
    return hipErrorInvalidValue;
  const dim3 g(max_items), b(256);
  if (a.fused) {
    if (a.w4)
      hipLaunchKernelGGL((expert_decode_kernel<kWFp4, true>), g, b, 0, s, a);
    else if (a.w8)
      hipLaunchKernelGGL((expert_decode_kernel<kWFp8, true>), g, b, 0, s, a);
    else
      hipLaunchKernelGGL((expert_decode_kernel<kWBf16, true>), g, b, 0, s, a);
  } else if (a.w4) {
    hipLaunchKernelGGL((expert_decode_kernel<kWFp4, false>), g, b, 0, s, a);
  } else if (a.w8) {
    hipLaunchKernelGGL((expert_decode_kernel<kWFp8, false>), g, b, 0, s, a);
  } else {
    hipLaunchKernelGGL((expert_decode_kernel<kWBf16, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine straight from the chunk partials.  A token's terms are its routes'
// chunk partials (routes in ascending expert id, each route's chunks in
// order) times the route's gate weight, then the shared row's chunk
// partials; term p is summed by chunk lane p % 16 in ascending p, the 16
// lane sums are added in lane order, then the residual source, one rounding
// ("NemotronH", "Arithmetic"; no atomics, so the result is deterministic).
// Grid: tokens x column blocks of 64; a thread owns 4 columns of one chunk
// lane, so a one-token batch still spreads its partials over d / 64
// workgroups.
// ---------------------------------------------------------------------------
constexpr int kCmbCols = 64, kCmbLanes = 16;

__global__ __launch_bounds__(256) void combine_decode_kernel(const float* __restrict__ part, int nc,
                                                             const float* __restrict__ w,
                                                             const int32_t* __restrict__ ids,
                                                             const int32_t* __restrict__ rpos, int K, int d,
                                                             const float* __restrict__ part_s, int ncs,
                                                             const void* resid, void* __restrict__ out,
                                                             int out_bf16) {
  __shared__ int s_pos[MOE_MAX_TOPK];
  __shared__ float s_w[MOE_MAX_TOPK];
  __shared__ float4 s_sum[kCmbLanes][kCmbCols / 4];
  const int t = blockIdx.x, tid = threadIdx.x, cl = tid & 15, q = tid >> 4;
  if (tid < 64) {
    const int k = tid;
    const int myid = k < K ? ids[(long)t * K + k] : 0x7fffffff;
    int rank = 0;
    for (int j = 0; j < K; ++j) rank += __shfl(myid, j, 64) < myid;
    if (k < K) {
      s_pos[rank] = rpos[(long)t * K + k];
      s_w[rank] = w[(long)t * K + k];
    }
  }
  __syncthreads();
  const int col = blockIdx.y * kCmbCols + cl * 4;
  const bool cin = col < d;
  const int nr = K * nc, np = nr + (part_s ? ncs : 0);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (cin) {
#pragma unroll 4
    for (int p = q; p < np; p += kCmbLanes) {
      const float* src;
      float g;
      if (p < nr) {
        const int j = p / nc, c = p - j * nc;
        src = part + ((long)s_pos[j] * nc + c) * d + col;
        g = s_w[j];
      } else {
        src = part_s + ((long)t * ncs + (p - nr)) * d + col;
        g = 1.0f;
      }
      const float4 v = *(const float4*)src;
      acc.x = fmaf(g, v.x, acc.x);
      acc.y = fmaf(g, v.y, acc.y);
      acc.z = fmaf(g, v.z, acc.z);
      acc.w = fmaf(g, v.w, acc.w);
    }
  }
  s_sum[q][cl] = acc;
  __syncthreads();
  if (q != 0 || !cin) return;
  float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int l = 0; l < kCmbLanes; ++l) {
    const float4 v = s_sum[l][cl];
    y[0] += v.x;
    y[1] += v.y;
    y[2] += v.z;
    y[3] += v.w;
  }
  const long o = (long)t * d + col;
  if (out_bf16) {
    if (resid) {
      const uint2 r = *(const uint2*)((const uint16_t*)resid + o);
      y[0] += bf16_to_f32(r.x & 0xffffu);
      y[1] += bf16_to_f32(r.x >> 16);
      y[2] += bf16_to_f32(r.y & 0xffffu);
      y[3] += bf16_to_f32(r.y >> 16);
    }
    *(uint2*)((uint16_t*)out + o) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
  } else {
    if (resid) {
      const float4 r = *(const float4*)((const float*)resid + o);
      y[0] += r.x;
      y[1] += r.y;
      y[2] += r.z;
      y[3] += r.w;
    }
    *(float4*)((float*)out + o) = make_float4(y[0], y[1], y[2], y[3]);
  }
}

hipError_t launch_combine_decode(const float* part, int nc, const float* w, const int32_t* ids,
                                 const int32_t* rpos, int T, int K, int d, const float* part_s,
                                 int ncs, const void* resid, void* out, int out_bf16, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (d % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_decode_kernel, dim3(T, ceil_div(d, kCmbCols)), dim3(256), 0, s, part, nc, w, ids, rpos,
                     K, d, part_s, ncs, resid, out, out_bf16);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Sum of each row's chunk partials: out[j] = sum_c part[j][c] for the routed
// rows and out_s[t] = sum_c part_s[t][c] for the shared rows, in a fixed
// order (eight interleaved partial sums, then added in order), so the
// result is deterministic.  Grid: (routed rows + shared rows) x column
// blocks of 256; a thread owns 8 columns of one of the 8 partial sums.
__global__ __launch_bounds__(256) void reduce_chunks_kernel(const float* __restrict__ part, int R, int nc,
                                                            int d, void* __restrict__ out, int out_bf16,
                                                            const float* __restrict__ part_s, int Ts,
                                                            int ncs, int ds, float* __restrict__ out_s) {
  __shared__ float s_sum[8][256];
  const int tid = threadIdx.x, cl = tid & 31, rgp = tid >> 5;
  const bool shared_row = (int)blockIdx.x >= R;
  const int j = shared_row ? blockIdx.x - R : blockIdx.x;
  const int n = shared_row ? ncs : nc, w = shared_row ? ds : d;
  const float* p = shared_row ? part_s : part;
  const int col = blockIdx.y * 256 + cl * 8;
  if (blockIdx.y * 256 >= w) return;  // uniform
  float y[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (col < w) {
    const float* pr = p + (long)j * n * w + col;
    for (int cc = rgp; cc < n; cc += 8) {
      const float4 a0 = *(const float4*)(pr + (long)cc * w), a1 = *(const float4*)(pr + (long)cc * w + 4);
      y[0] += a0.x; y[1] += a0.y; y[2] += a0.z; y[3] += a0.w;
      y[4] += a1.x; y[5] += a1.y; y[6] += a1.z; y[7] += a1.w;
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) s_sum[rgp][cl * 8 + q] = y[q];
  __syncthreads();
  if (rgp != 0 || col >= w) return;
  float z[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    float t = s_sum[0][cl * 8 + q];
#pragma unroll
    for (int g = 1; g < 8; ++g) t += s_sum[g][cl * 8 + q];
    z[q] = t;
  }
  const long o = (long)j * w + col;
  if (shared_row || !out_bf16) {
    float* po = shared_row ? out_s + o : (float*)out + o;
    *(float4*)po = make_float4(z[0], z[1], z[2], z[3]);
    *(float4*)(po + 4) = make_float4(z[4], z[5], z[6], z[7]);
  } else {
    *(uint4*)((uint16_t*)out + o) = make_uint4(pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3]),
                                               pack_bf16x2(z[4], z[5]), pack_bf16x2(z[6], z[7]));
  }
}

hipError_t launch_reduce_chunks(const float* part, int R, int nc, int d, void* out, int out_bf16,
                                const float* part_s, int Ts, int ncs, int ds, float* out_s,
                                hipStream_t s) {
  const int rows = R + (part_s ? Ts : 0);
  if (rows <= 0) return hipSuccess;
  const int cb = ceil_div(max(d, part_s ? ds : 0), 256);
  hipLaunchKernelGGL(reduce_chunks_kernel, dim3(rows, cb), dim3(256), 0, s, part, R, nc, d, out, out_bf16,
                     part_s, Ts, ncs, ds, out_s);
  return hipGetLastError();
}

}  // namespace moe
