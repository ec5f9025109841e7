// Internal declarations of libmoe: device helpers shared by the kernels and
// the host-side launchers called by the C ABI in moe_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

#include <math.h>

#include <algorithm>

namespace moe {

// ---------------------------------------------------------------------------
// bf16 helpers (bf16 = upper 16 bits of an IEEE binary32)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t v16) {
  return __uint_as_float(v16 << 16);
}
// round to nearest even (the CDNA4 v_cvt_pk_bf16_f32 conversion); NaN stays NaN
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// two values rounded to bf16 and packed, lo in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ float bf16_round(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// ---------------------------------------------------------------------------
// FP8 (OCP E4M3) weights.  The CDNA4 conversions decode the OCP format
// exactly (every E4M3 value, subnormals included, is a bf16 and an fp32
// value; a unit scale leaves it unchanged).
// ---------------------------------------------------------------------------
// Eight codes (the bytes of v, lowest first) as eight bf16, packed lo-first.
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint2 v) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true);
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                    __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
}
// Eight codes as eight fp32 values.
__device__ __forceinline__ void fp8x8_to_f32(uint2 v, float (&f)[8]) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(v.x, false);
  const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(v.x, true);
  const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8(v.y, false);
  const f32x2_t d = __builtin_amdgcn_cvt_pk_f32_fp8(v.y, true);
  f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
  f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
}

// MXFP4: the E8M0 scale byte e as the fp32 value 2^(e - 127) (e = 0 is the
// subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
}
// Eight E2M1 codes (one 32-bit word; element 2i in the low nibble of byte i)
// times a scale 2^k, as eight bf16 (exact: an E2M1 value has at most two
// significant bits).
__device__ __forceinline__ uint4 fp4x8_to_bf16x8(uint32_t v, float s) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 0);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 1);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 2);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 3);
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                    __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
}
// Eight E2M1 codes as eight fp32 values (unscaled).
__device__ __forceinline__ void fp4x8_to_f32(uint32_t v, float (&f)[8]) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 0);
  const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 1);
  const f32x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 2);
  const f32x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 3);
  f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
  f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
}
constexpr int kMxBlock = 32;  // MXFP4 elements per scale

// ---------------------------------------------------------------------------
// One router row per wave (route_kernel, and the fused small-batch decode
// kernel): s = sigmoid(z), c = s + bias; groups of E / n_group scored by
// their two largest c, the topk_group best kept (equal scores: lower group);
// the K largest c among the kept experts in descending order (equal c: lower
// id); weights s[id], normalised to sum 1 when `norm`, times rsf.  Lane l
// holds experts l*VPL .. l*VPL+VPL-1; s_sig / s_cor are the wave's LDS rows
// (VPL * 64 floats each).  Contains a __syncthreads(): every wave of the
// workgroup calls it the same number of times.  Lanes < K receive the row's
// k-th id and weight.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t route_orderable(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Maximum of v over the wave, returned to every lane (a scalar).  Within each
// row of 16 lanes DPP moves fold quads (lane ^ 1, lane ^ 2), then half rows
// (mirror within 8 lanes), then rows (mirror within 16 lanes); the four row
// maxima are read out with v_readlane.  No LDS round trip.
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v, int ctrl_sel) {
  int o;
  switch (ctrl_sel) {
    case 0: o = __builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false); break;   // quad_perm [1,0,3,2]
    case 1: o = __builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false); break;   // quad_perm [2,3,0,1]
    case 2: o = __builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    default: o = __builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false); break; // row_mirror
  }
  return max(v, (uint32_t)o);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) v = dpp_max_u32(v, i);
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// The wave's largest key and the lowest lane holding it (keys of 0 never
// win unless every key is 0; then lane 0).
__device__ __forceinline__ int wave_argmax_lane(uint32_t key, uint32_t* best) {
  const uint32_t m = wave_max_u32(key);
  const unsigned long long hit = __ballot(key == m);
  *best = m;
  return hit ? __builtin_ctzll(hit) : 0;
}

template <int VPL>
__device__ __forceinline__ void route_row(const float* __restrict__ logits, int S, long sstride,
                                          const float* __restrict__ bias, long t, bool valid, int E, int K,
                                          int n_group, int topk_group, int norm, float rsf, float* s_sig,
                                          float* s_cor, int lane, int* out_id, float* out_w) {
  float cv[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = lane * VPL + v;
    float sg = 0.0f, c = -INFINITY;
    if (valid && e < E) {
      const long idx = t * E + e;
      float z = logits[idx];
#pragma unroll 4
      for (int k = 1; k < S; ++k) z += logits[k * sstride + idx];
      sg = 1.0f / (1.0f + expf(-z));
      c = sg + (bias ? bias[e] : 0.0f);
    }
    cv[v] = c;
    s_sig[e] = sg;
    s_cor[e] = c;
  }
  __syncthreads();

  // group selection: lane g scores group g by its two largest corrected scores
  unsigned long long gmask = ~0ull;
  const int gs = E / n_group;
  if (n_group > 1) {
    // group g's key: its score's order-preserving bits (lane g); the
    // largest key wins, equal keys go to the lower group (lower lane)
    uint32_t key = 0;
    if (lane < n_group) {
      float m1 = -INFINITY, m2 = -INFINITY;
      for (int i = 0; i < gs; ++i) {
        const float c = s_cor[lane * gs + i];
        if (c > m1) {
          m2 = m1;
          m1 = c;
        } else if (c > m2) {
          m2 = c;
        }
      }
      key = max(route_orderable(m1 + m2), 1u);
    }
    gmask = 0;
    for (int r = 0; r < topk_group; ++r) {
      uint32_t best;
      const int g = wave_argmax_lane(key, &best);
      gmask |= 1ull << g;
      if (lane == g) key = 0;
    }
  }

  // expert e's key: its corrected score's order-preserving bits, 0 when it
  // is not eligible (an eligible key is at least 1); the largest key wins,
  // equal keys go to the lower id: the lowest lane holding the maximum, and
  // within that lane the lower slot (e = lane * VPL + v)
  uint32_t keys[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = lane * VPL + v;
    const bool elig = e < E && ((gmask >> (e / gs)) & 1ull);
    keys[v] = elig ? max(route_orderable(cv[v]), 1u) : 0u;
  }

  int my_id = 0;
  float my_s = 0.0f, wsum = 0.0f;
  for (int r = 0; r < K; ++r) {
    uint32_t m = 0;
    int mv = 0;
#pragma unroll
    for (int v = 0; v < VPL; ++v)
      if (keys[v] > m) {
        m = keys[v];
        mv = v;
      }
    uint32_t best;
    const int wl = wave_argmax_lane(m, &best);
    const int wv = __builtin_amdgcn_readlane(mv, wl);
    const int e = wl * VPL + wv;
    if (lane == wl)
#pragma unroll
      for (int v = 0; v < VPL; ++v)
        if (v == wv) keys[v] = 0u;
    const float sg = s_sig[e];
    wsum += sg;
    if (lane == r) {
      my_id = e;
      my_s = sg;
    }
  }
  const float w = norm ? my_s / wsum : my_s;
  *out_id = my_id;
  *out_w = w * rsf;
}

// ---------------------------------------------------------------------------
// Tile plan of the grouped GEMMs.
//
// A grouped GEMM launch covers group 0 (a dense "shared" group of M_s rows,
// possibly empty) and groups 1..E (routed expert e = g-1, rows
// [offsets[e], offsets[e+1]) of the packed route space).  Each group is cut
// into row chunks of kChunkRows rows and column tiles of kTileN columns.
// The plan lists every (group, chunk, column tile) as two int32:
//   plan[2t] = group, plan[2t+1] = (chunk << 16) | ntile,
// groups in order 0..E, and inside a group blocks of kChunkBlock chunks
// walked column tile by column tile, so tiles that run at the same time on
// one XCD share their weight tile (same ntile) or their rows (same chunk).
// ---------------------------------------------------------------------------
constexpr int kChunkRows = 256;
constexpr int kTileN = 256;
// Tiles of dense launches of the split-K kernel (the router GEMM).
constexpr int kDenseChunkRows = 128;
constexpr int kDenseTileN = 128;
constexpr int kChunkBlock = 8;
// Launch-order blocks: kXcdBlock consecutive plan tiles run on one XCD.
constexpr int kXcdBlock = 16;
constexpr int kNumXcd = 8;

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ inline int imin(int a, int b) { return a < b ? a : b; }

// ---------------------------------------------------------------------------
// Packed weight layout (moe_pack_weight).  One matrix W [R][C] keeps R * C
// elements, rearranged so that one K step of the grouped GEMM reads one
// contiguous range:
//  * [out][in] matrices (up projections, latent projections; R = out,
//    C = in): rows in tiles of kPackTile (the last tile rn = R - r0 rows),
//    each tile stored as its K steps of kPackStep columns (the last step
//    kw = C - c0 <= kPackStep columns), a step a row-major [rn][kw] block;
//  * neuron-major down matrices (R = hidden neurons, C = outputs): columns in
//    strips of kPackTile (the last strip cn = C - c0 columns), each strip a
//    row-major [R][cn] block, so the 32 neurons of a K step are one range and
//    a neuron's outputs inside a strip are contiguous.
// ---------------------------------------------------------------------------
constexpr int kPackTile = 256;
constexpr int kPackStep = 32;
__host__ __device__ inline long packed_out_in_offset(int r, int c, int R, int C) {
  const int r0 = r & ~(kPackTile - 1);
  const int rn = imin(kPackTile, R - r0);
  const int c0 = c & ~(kPackStep - 1);
  const int kw = imin(kPackStep, C - c0);
  return (long)r0 * C + (long)c0 * rn + (long)(r - r0) * kw + (c - c0);
}
__host__ __device__ inline long packed_neuron_major_offset(int r, int c, int R, int C) {
  const int c0 = c & ~(kPackTile - 1);
  const int cn = imin(kPackTile, C - c0);
  return (long)c0 * R + (long)r * cn + (c - c0);
}

// Decode local tile l of a group with nch chunks and ntc column tiles.
__host__ __device__ inline void plan_decode_local(int l, int nch, int ntc, int* ch, int* nt) {
  int blk = kChunkBlock * ntc;
  int cb = l / blk;
  int within = l - cb * blk;
  int w = nch - cb * kChunkBlock;
  if (w > kChunkBlock) w = kChunkBlock;
  *nt = within / w;
  *ch = cb * kChunkBlock + (within - (within / w) * w);
}

// The plan tile index handled by workgroup `wg` (XCD-blocked order: WGs are
// dealt round-robin to the 8 XCDs, so XCD x receives WGs x, x+8, ...; give
// it whole blocks of kXcdBlock consecutive tiles).
__host__ __device__ __forceinline__ int xcd_tile_of(int wg) {
  int x = wg % kNumXcd;
  int s = wg / kNumXcd;
  return ((s / kXcdBlock) * kNumXcd + x) * kXcdBlock + (s % kXcdBlock);
}
// Grid size covering max_tiles plan tiles under xcd_tile_of.
inline int xcd_grid(int max_tiles) {
  int per = kNumXcd * kXcdBlock;
  return ceil_div(max_tiles > 0 ? max_tiles : 1, per) * per;
}

// The weight-gradient launches' order (E experts of tpr tiles, after tps
// tiles of group 0): XCD x takes a contiguous eighth of group 0's tiles and
// then whole experts x, x + 8, ..., so an expert's two operand panels (its
// rows of both transposed matrices) are read into one XCD's L2 once and
// serve all of its tiles there.  Returns the tile index (group 0: [0, tps),
// expert e: tps + e tpr + l) or -1.
__host__ __device__ __forceinline__ int wgrad_tile_of(int wg, int E, int tpr, int tps) {
  const int x = wg % kNumXcd, slot = wg / kNumXcd;
  const int q = (tps + kNumXcd - 1) / kNumXcd;
  const int s0 = x * q < tps ? x * q : tps;
  const int ns = (s0 + q < tps ? s0 + q : tps) - s0;
  if (slot < ns) return s0 + slot;
  if (tpr == 0) return -1;
  const int r = slot - ns, j = r / tpr;
  const int e = j * kNumXcd + x;
  return e < E ? tps + e * tpr + (r - j * tpr) : -1;
}
// Grid size of a weight-gradient launch under wgrad_tile_of.
inline int wgrad_grid(int E, int tpr, int tps) {
  return kNumXcd * ((tps + kNumXcd - 1) / kNumXcd + (E + kNumXcd - 1) / kNumXcd * tpr);
}

struct PlanSpec {
  int E;          // routed groups
  int M_s;        // rows of group 0 (0 = none)
  int ntc_r;      // column tiles of routed groups
  int ntc_s;      // column tiles of group 0
};

// Upper bound on the tiles of a plan with R routed rows.
inline long plan_max_tiles(const PlanSpec& p, long R) {
  long ch_r = R / kChunkRows + p.E;  // sum over experts of ceil(c_e / kChunkRows)
  long rmax = (R + kChunkRows - 1) / kChunkRows;
  if (ch_r > rmax + p.E) ch_r = rmax + p.E;
  return ch_r * p.ntc_r + (long)ceil_div(p.M_s, kChunkRows) * p.ntc_s;
}

// ---------------------------------------------------------------------------
// Grouped GEMM arguments.
//   C[row, n] = sum_k A[row', k] * B_g[n, k]   (B stored [N][K], "NK")
//   or          sum_k A[row', k] * B_g[k, n]   (B stored [K][N], "KN")
// Routed group g >= 1 (expert e = g-1): packed rows j in
// [offsets[e], offsets[e+1]); A row = gather ? gather[j] / gdiv : j; output
// row j.  Group 0: rows 0..M_s-1, A_s / B_s / C_s.
// ---------------------------------------------------------------------------
// EPI_DRELU2 (backward of ReLU^2): C = round(acc * 2 sqrt(aux[row, n])), aux
// the bf16 h = relu(u)^2 of the forward (C's row stride), so 2 sqrt(h) is
// ReLU^2's derivative 2 relu(u) up to h's rounding.
// EPI_QRELU2 (the MX kernel): relu(acc)^2 in fp32, quantised to MXFP8 (E4M3
// codes and an E8M0 scale per 32 columns of a row).
enum { EPI_RELU2 = 0, EPI_STORE = 1, EPI_ADD_F32 = 2, EPI_DRELU2 = 3, EPI_QRELU2 = 4 };
// B_NKP: B stored plain row-major [N][ldb], K contiguous (not packed).
enum { B_NK = 0, B_KN = 1, B_NKP = 2 };

struct GemmArgs {
  // routed groups
  int E;
  const int32_t* offsets;
  const int32_t* gather;
  int gdiv;
  const void* A;
  long lda;
  const void* B;
  long strideB;  // elements between consecutive experts' matrices
  long ldb;      // elements between rows of one expert's matrix
  int N, Kd;
  void* C;
  long ldc;
  int c_f32;
  // group 0
  int M_s;
  const void* A_s;
  long lda_s;
  const void* B_s;
  long ldb_s;
  int N_s, Kd_s;
  void* C_s;
  long ldc_s;
  int c_s_f32;
  // EPI_ADD_F32: C = round(acc + addend[row, n] (+ resid[row, n])); resid
  // (C's dtype and row stride, may be C itself) is the residual / old output
  const float* addend;
  long ld_add;
  const void* resid;
  // plan (routed launches) or NULL for a dense group-0-only launch
  const int32_t* plan;
  const int32_t* num_tiles;  // device scalar
  // dense launches only: split the K loop into ksplit parts, part p writing
  // C_s + p * split_stride; A columns repeat with period a_period (0 = no
  // repeat), so B may be several K-concatenated planes applied to one A.
  int ksplit;
  long split_stride;
  int a_period;
  int a_cols;  // with a_period: A columns [a_cols, a_period) read as zero
  // B of both groups in the packed layout (packed_out_in_offset for B_NK,
  // packed_neuron_major_offset for B_KN); the bf16 tile kernel requires it
  int b_packed;
  // B of both groups as FP8 (E4M3) codes with fp32 scales per output
  // column n: bscale [E][N] (routed), bscale_s [N_s] (group 0); the tile
  // kernel multiplies the fp32 sum by the scale before the epilogue
  int b_fp8;
  const float* bscale;
  const float* bscale_s;
  // MXFP4 B (B_NK): E8M0 scales, block-major: e8 [E][Kd / 32][N] (routed),
  // e8_s [Kd_s / 32][N_s] (group 0); applied to the codes before the MFMA
  int b_fp4;
  const uint8_t* e8;
  const uint8_t* e8_s;
  // dense launches with ksplit > 1 on the main (256 x 256) kernel instead of
  // the 128 x 128 split-K kernel: fp32 partials at C_s + ks * split_stride,
  // summed by launch_reduce_splits
  int split_main;
  // EPI_DRELU2: h of the routed rows / of group 0 (bf16, C's layout)
  const void* aux;
  const void* aux_s;
  // weight-gradient launches (plan == NULL, wgrad != 0, B_NKP, fp32 C):
  // C_g = A_g B_g^T, the reduction running over the columns of group g.
  // Routed group g >= 1 (expert e = g - 1): A = A + koff[e] (M rows of
  // stride lda), B = B + koff[e] (N rows of stride ldb), K = koff[e+1] -
  // koff[e] (a multiple of 8, the columns past the group's rows zero),
  // C = C + e * M * N (ldc = N).  Group 0 (when Kd_s > 0): A_s, B_s, C_s
  // with M_s rows, N_s columns and K = Kd_s.
  int wgrad;
  int M;
  const int32_t* koff;
  // MXFP8 A (the MX kernel, gemm_mx_kernel): A holds E4M3 codes (lda bytes
  // per row) with E8M0 scales block-major, the scale of A row r (its packed
  // row for a routed group, its row for group 0), block j at
  // as[j * ld_as + r] (as_s / ld_as_s for group 0); ld_as a multiple of 4
  // with 256 bytes of slack past the last row
  const uint8_t* as;
  const uint8_t* as_s;
  long ld_as, ld_as_s;
  // EPI_QRELU2 output: C holds E4M3 codes of relu(acc)^2 (ldc bytes per
  // row), their E8M0 scales block-major at cs[j * ld_cs + row] (cs_s /
  // ld_cs_s for group 0)
  uint8_t* cs;
  uint8_t* cs_s;
  long ld_cs, ld_cs_s;
};

// ---------------------------------------------------------------------------
// Launchers (all asynchronous on `s`; return hipGetLastError()).
// ---------------------------------------------------------------------------
hipError_t launch_router_gemm_f32(const void* x, int x_bf16, int T, int d, const float* w,
                                  int E, float* logits, hipStream_t s);
// bf16 x: W_r is split into three bf16 planes hi + mid + lo == W_r exactly,
// stored K-concatenated as w3 [E][3 dp] (dp = d rounded up to 64, pad
// columns zero); split-K partial logits [S][T][E].
inline int router_plane_width(int d) { return (d + 63) / 64 * 64; }
int router_bf16_splits(int T, int d, int E);
hipError_t launch_split_router_weight(const float* w, int E, int d, uint16_t* w3, hipStream_t s);
hipError_t launch_router_gemm_bf16x3(const uint16_t* x, int T, int d, const uint16_t* w3, int E,
                                     float* partials, int S, hipStream_t s);
hipError_t launch_sum_partials(const float* partials, int S, long n, float* out, hipStream_t s);
hipError_t launch_route(const float* logits, int S, const float* bias, int T, int E, int K,
                        int n_group, int topk_group, int norm, float rsf, int32_t* ids,
                        float* weights, hipStream_t s);

size_t dispatch_scratch_bytes(int T, int E);
struct PlanOut {
  int32_t* plan_up;
  int32_t* plan_down;
  int32_t* num_tiles;  // [2]: up, down
  PlanSpec up, down;
};
hipError_t launch_dispatch(const int32_t* ids, int T, int K, int E, int32_t* counts,
                           int32_t* offsets, int32_t* route_src, int32_t* route_pos,
                           void* scratch, const PlanOut* plan, hipStream_t s);
hipError_t launch_plan(const int32_t* offsets, const PlanOut* plan, hipStream_t s);
// Fixed capacity over a dropless dispatch (counts_all, offsets_all, src_all):
// accepted counts/offsets/route_src, route_pos = -1 for overflowed routes.
hipError_t launch_capacity(const int32_t* counts_all, const int32_t* offsets_all, const int32_t* src_all,
                           const float* gates, int E, int C, int32_t* counts, int32_t* offsets,
                           int32_t* route_src, int32_t* route_pos, hipStream_t s);

hipError_t launch_gemm(const GemmArgs& a, int act_bf16, int b_mode, int epi, int max_tiles,
                       hipStream_t s);
// MXFP8 A x MXFP4 B grouped GEMM on the block-scaled MFMA (B packed
// [OUT_IN] MXFP4 codes with block-major scales e8 / e8_s; epi EPI_QRELU2 or
// EPI_STORE).
hipError_t launch_gemm_mx(const GemmArgs& a, int epi, int max_tiles, hipStream_t s);
// MXFP8 quantisation of bf16 rows x [T][W] (W a multiple of 32): codes
// [T][W] and E8M0 scales block-major, scales [j][t] (ld_s per block row).
hipError_t launch_quantize_act_mxfp8(const uint16_t* x, int T, int W, uint8_t* codes, uint8_t* scales, long ld_s,
                                     hipStream_t s);
// Token-order MXFP8 scales [W/32][ld_t] -> packed-row order [W/32][ld_r] for
// the first *n_rows packed rows (row p takes token route_src[p] / K).
hipError_t launch_gather_mx_scales(const uint8_t* tok, long ld_t, const int32_t* route_src, const int32_t* n_rows,
                                   int K, int W, int R, uint8_t* packed, long ld_r, hipStream_t s);
// The scale-matrix row stride of the MX activation operands for `rows` rows.
inline long mx_scale_ld(long rows) { return (rows + 3) / 4 * 4 + 256; }
// Backward pass (backward.hip).
hipError_t launch_gate_grad(const uint16_t* dy, const float* U, const float* logits, int S, long sstride,
                            const int32_t* ids, const float* gates, const int32_t* rpos, int T, int E, int K, int d,
                            int norm, float rsf, float* dz, uint16_t* dU, hipStream_t s);
hipError_t launch_router_grad(const uint16_t* x, int d, int K, int E, const int32_t* offsets,
                              const int32_t* route_src, const float* dz, float* dw, hipStream_t s);
hipError_t launch_dx_combine(const float* dxp, const float* dx_s, const float* dx_s2, const float* w_router,
                             const int32_t* ids, const int32_t* rpos, const float* dz, int T, int K, int d,
                             uint16_t* dx, float* dx32, hipStream_t s);
hipError_t launch_wgrad_map(const int32_t* offsets, const int32_t* route_src, int E, int K, int Rp, int32_t* koff,
                            int32_t* row_of, int32_t* tok_of, hipStream_t s);
hipError_t launch_transpose_rows(const uint16_t* in, long ldi, int C, const int32_t* map, int nsrc, int ncol,
                                 uint16_t* out, long ldo, hipStream_t s);
// Per-row FP8 (E4M3) quantisation of [rows][C] weights: codes and fp32 scales.
hipError_t launch_quantize_mxfp4(const void* w, int bf16, int G, int R, int C, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s);
hipError_t launch_quantize_fp8(const void* w, int bf16, long rows, int C, uint8_t* codes, float* scales,
                               hipStream_t s);
// Rearrange [G][R][C] matrices (plain row-major) into the packed layout.
hipError_t launch_pack_weight(const void* src, int elem_bytes, int neuron_major, int G, int R, int C,
                              void* dst, hipStream_t s);

// ---------------------------------------------------------------------------
// Decode-size batches: fused up + ReLU^2 + zero-skipping down per
// (group, 64-neuron chunk) item, fp32 partial outputs, deterministic combine.
// ---------------------------------------------------------------------------
constexpr int kDecodeMaxRows = 256;     // rows of one group (and T) on this path
constexpr int kDecodeMaxRoutes = 8192;  // T * K handled by the one-workgroup dispatch
constexpr int kDecodeChunk = 64;        // hidden neurons per work item
constexpr int kDecodeItemRows = 16;     // group rows per work item
// Upper bound on the work items of R routes over E experts (rows split in
// blocks of kDecodeItemRows) plus a shared group of Ts rows.
inline long decode_max_items(int E, long R, int ncr, int Ts, int ncs) {
  const long blocks = std::min<long>(E, R) + R / kDecodeItemRows;
  return blocks * ncr + (long)((Ts + kDecodeItemRows - 1) / kDecodeItemRows) * ncs;
}
constexpr int kDecodeMaxWidth = 4096;   // output width: 2 x 8-column groups per thread of 256
// Batches the fused decode kernel routes and dispatches itself (every
// workgroup, in LDS): at most kFusedRows rows, kFusedExperts experts.
constexpr int kFusedRows = 8;
constexpr int kFusedExperts = 128;

struct DecodeArgs {
  // routed groups 0..E-1 (expert e: packed rows [offsets[e], offsets[e+1]))
  int E, K;
  const int32_t* offsets;
  const int32_t* route_src;  // packed row -> route t*K+k; NULL: packed row j reads x row j
  const uint16_t* x;         // [*, d_e] bf16
  long ldx;
  int d_e, F;
  const void* w_up;          // [E][F][d_e]  bf16, or FP8 codes with w8
  const void* w_dn;          // [E][F][d_e] neuron-major
  float* part;               // [R][ncr][d_e] fp32 partial outputs
  int ncr;                   // ceil(F / kDecodeChunk)
  // shared group E (M_s rows = x_s rows 0..M_s-1; M_s = 0: none)
  int M_s;
  const uint16_t* x_s;
  long ldx_s;
  int d_s, F_s;
  const void* w_up_s;        // [F_s][d_s]
  const void* w_dn_s;        // [F_s][d_s] neuron-major
  float* part_s;             // [M_s][ncs][d_s]
  int ncs;
  // work items: (group << 16) | chunk
  const int32_t* items;
  const int32_t* n_items;
  unsigned long long* zero_count;  // NULL or [2] (+[2] for the shared group): zeros, skipped rows
  // fused small batches (route and dispatch inside every workgroup): the
  // router logits [T][E] and the routing parameters in; workgroup 0 writes
  // ids, weights and route_pos for the combine, and the counts, offsets and
  // route_src of the same dispatch
  int fused;
  int T;
  const float* logits;
  const float* bias;
  int n_group, topk_group, norm;
  float rsf;
  int32_t* ids_out;
  float* wts_out;
  int32_t* rpos_out;
  int32_t* counts_out;
  int32_t* offsets_out;
  int32_t* src_out;
  // FP8 expert weights: per-neuron up scales and per-output down scales
  int w8;
  const float* s_up;    // [E][F]
  const float* s_dn;    // [E][d_e]
  const float* s_up_s;  // [F_s]
  const float* s_dn_s;  // [d_s]
  // MXFP4 expert weights: E8M0 scales, block-major
  int w4;
  const uint8_t* e_up;    // [E][d_e / 32][F]
  const uint8_t* e_dn;    // [E][F / 32][d_e]
  const uint8_t* e_up_s;  // [d_s / 32][F_s]
  const uint8_t* e_dn_s;  // [F_s / 32][d_s]
};
hipError_t launch_router_small(const uint16_t* x, int T, int d, const float* w, int E, float* logits,
                               hipStream_t s);
hipError_t launch_dispatch_small(const int32_t* ids, int T, int K, int E, int32_t* counts,
                                 int32_t* offsets, int32_t* route_src, int32_t* route_pos, int ncr,
                                 int ncs, int32_t* items, int32_t* n_items, hipStream_t s);
hipError_t launch_decode_items(const int32_t* offsets, int E, int ncr, int32_t* items,
                               int32_t* n_items, hipStream_t s);
hipError_t launch_expert_decode(const DecodeArgs& a, int max_items, hipStream_t s);
hipError_t launch_combine_decode(const float* part, int nc, const float* w, const int32_t* ids,
                                 const int32_t* rpos, int T, int K, int d, const float* part_s,
                                 int ncs, const void* resid, void* out, int out_bf16, hipStream_t s);
// out[j] = sum_c part[j][c] (j < R, in bf16 or fp32) and out_s[t] = sum_c
// part_s[t][c] (t < Ts, fp32; part_s may be NULL), in a fixed order.
hipError_t launch_reduce_chunks(const float* part, int R, int nc, int d, void* out, int out_bf16,
                                const float* part_s, int Ts, int ncs, int ds, float* out_s,
                                hipStream_t s);

hipError_t launch_combine(const void* y_packed, int act_bf16, const float* weights,
                          const int32_t* ids, const int32_t* route_pos, const float* y_shared,
                          int T, int K, int d, const void* resid, void* out, hipStream_t s);
// out[r][c] = round(sum_s part[s][r][c] + addend[r][c] + resid[r][c]) for
// r < rows, c < N (part: S slices of rows x N fp32, split_stride apart;
// addend fp32 with row stride ld_add, or NULL; resid in the output's dtype,
// row stride N, or NULL), the slices summed in order, one rounding.
hipError_t launch_reduce_splits(const float* part, int S, long split_stride, int rows, int N, const float* addend,
                                long ld_add, const void* resid, void* out, int out_bf16, hipStream_t s);
// The combine with fp32 packed rows and a bf16 output (the training forward).
hipError_t launch_combine_y32(const float* y_packed, const float* weights, const int32_t* ids,
                              const int32_t* route_pos, const float* y_shared, int T, int K, int d,
                              const void* resid, void* out, hipStream_t s);
// Backward of the fused front (bf16): dh = dy + RMSNorm'(h)^T dx (rounded
// to bf16), dw = sum over rows of dx * h / rms (fp32); r_buf [T] and part
// [rmsnorm_dw_blocks(T)][d] are scratch.
int rmsnorm_dw_blocks(int T);
hipError_t launch_rmsnorm_bwd(const uint16_t* h, const uint16_t* w, float eps, int T, int d, const float* dx,
                              const uint16_t* dy, uint16_t* dh, float* dw, float* r_buf, float* part,
                              hipStream_t s);
// y = RMSNorm(x) * w per row in fp32, rounded once to the activation dtype.
hipError_t launch_rmsnorm(const void* x, const void* w, float eps, int T, int d, int bf16, void* y,
                          hipStream_t s);

}  // namespace moe
