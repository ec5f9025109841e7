// MXFP8 x MXFP4 grouped GEMMs on CDNA4's block-scaled MFMA, for the W4A8
// expert variant: the routed and shared experts' inputs are MXFP8 (OCP MX:
// E4M3 codes, one E8M0 scale per 32 values along K) and their weights MXFP4
// (E2M1 codes, one E8M0 scale per 32 inputs).  The 8 GB Super write-up
// ("The only number that matters: bytes per token") and NemotronH ("How the
// engine runs it") serve the experts from 4-bit block-scaled checkpoints;
// here the activations are block-scaled too, so the product runs on
// v_mfma_scale_f32_32x32x64_f8f6f4, which applies both operands' block
// scales inside the MFMA (A FP8 E4M3, B FP4 E2M1), fp32 accumulation.
//
// Tile and waves as the bf16 kernel (gemm.hip): 256 x 256 per workgroup of 8
// waves (2 x 4), each wave 128 x 64 as 4 x 2 blocks of 32 x 32; rows
// gathered through the route map (up) or contiguous (down); the tile plan
// and its XCD-aware order are the same.  One K step is 64: the MFMA's K and
// two scale blocks.  A ring of 5 LDS stages of 30 KB is filled by direct
// global->LDS loads, 6 per wave and step (uniform, so one vmcnt count covers
// every wave), issued 4 steps ahead:
//  * A codes: 256 rows x 64 bytes, 16-byte chunk c of row r at position
//    c ^ ((r >> 2) & 3) (the bf16 kernel's A geometry and swizzle); a lane
//    of half h = lane >> 5 reads chunks h and 2 + h (see the operand layout
//    below);
//  * B codes: 256 rows x 32 bytes (two packed K steps of 16 bytes), half h
//    of row n at position h ^ ((n >> 3) & 1); a lane reads 16 bytes (32 FP4
//    codes of its column and k half);
//  * scales: each wave copies the ones it reads into its own 768 bytes:
//    its 128 rows' A scales of the step's two blocks (a 4-byte-aligned
//    window of the block-major scale rows, so the DMA reads whole dwords)
//    and its 64 columns' B scales of both blocks.
// A lane's MFMA operands (lane l, half h = l / 32; measured on the card with
// an in-bounds probe of single products): A row l % 32 of the block, its 8
// dwords of E4M3 holding k = 16h .. 16h + 15 (bytes 0-15) and k = 32 + 16h
// .. 32 + 16h + 15 (bytes 16-31); B column l % 32, 4 dwords of E2M1 codes
// holding k = 32h .. 32h + 31 (the upper 4 dwords zero); each lane's scale
// byte is the scale of K block h (k = 32h .. 32h + 31) of its row or column.
//
// Epilogues: EPI_QRELU2 (up projections) squares the ReLU in fp32 and
// quantises each row's 32-column blocks to MXFP8 for the down projection:
// the wave stages its fp32 block rows in LDS (68-float rows: conflict-free
// 16-byte reads), then each lane takes a (row, block), finds the block's
// amax, the shared exponent floor(log2 amax) - 8 and the 32 E4M3 codes
// (nearest, ties to even, saturating at 448), and stores 32 bytes of codes
// and one scale byte.  EPI_STORE (down projections): bf16 rows through LDS
// (16-byte stores) or fp32 (the shared expert's rows).
#include "moe_internal.h"
#include "tile.h"

namespace moe {

namespace {
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kMxWaveN = 4;
constexpr int kMxWaves = 8;
constexpr int kMxThreads = kMxWaves * 64;
constexpr int kMxBK = 64;                          // K per step
constexpr int kMxARow = 64;                        // A code bytes per tile row and step
constexpr int kMxAStage = kChunkRows * kMxARow;    // 16 KB
constexpr int kMxBRow = 32;                        // B code bytes per tile row and step
constexpr int kMxBStage = kTileN * kMxBRow;        // 8 KB
constexpr int kMxSWave = 768;                      // a wave's scales: A block 0, A block 1, B
constexpr int kMxStageBytes = kMxAStage + kMxBStage + kMxWaves * kMxSWave;  // 30 KB
constexpr int kMxStages = 5;
constexpr int kMxLoads = 6;                        // DMA loads per wave per step
constexpr int kMxRing = kMxStages * kMxStageBytes;
constexpr int kMxEpiRow = 68;                      // fp32 per staged row (64 + 4 pad)
constexpr int kMxEpiQ = kMxWaves * 64 * kMxEpiRow * 4;   // EPI_QRELU2: 64 rows per wave per pass
constexpr int kMxEpiS = kMxWaves * 128 * 64 * 2;         // EPI_STORE: the wave's bf16 block
constexpr int kMxSmem = kMxRing > kMxEpiQ ? (kMxRing > kMxEpiS ? kMxRing : kMxEpiS)
                                          : (kMxEpiQ > kMxEpiS ? kMxEpiQ : kMxEpiS);
static_assert(kMxSmem <= 160 * 1024, "fits the LDS of a CU");
static_assert(kMxStages - 2 <= 3, "the vmcnt waits cover at most 3 later steps in flight");
static_assert(kMxLoads * 3 < 64, "vmcnt counts up to 63");

__device__ __forceinline__ f32x16_t mfma_mx(const i32x8_t& a, const i32x8_t& b, uint32_t sa, uint32_t sb,
                                            f32x16_t c) {
  // A: FP8 E4M3 (format 0), B: FP4 E2M1 (format 4); scales in byte 0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 4, 0, (int)sa, 0, (int)sb);
}
}  // namespace

// The E4M3 code nearest to v (ties to the even code), magnitudes at or past
// 448 saturating to 448; -0 keeps its sign.  v finite.  Branch-free: both
// the normal and the subnormal rounding are computed and one is selected.
__device__ __forceinline__ uint32_t e4m3_encode_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(v);
  const uint32_t ua = u & 0x7FFFFFFFu;
  // normal binades: round the mantissa to 3 bits, ties to even; r >> 20 is
  // then (biased exponent << 3) | mantissa, and rebiasing 127 -> 7 takes
  // 120 << 3 off
  const uint32_t r = (ua + 0x7FFFFu + ((ua >> 20) & 1u)) & ~0xFFFFFu;
  const uint32_t nrm = (r >> 20) - (120u << 3);
  // subnormal range (below 2^-6): steps of 2^-9 (a * 512 is exact); 8
  // steps is 2^-6, the smallest normal, code 0x08
  const uint32_t sub = (uint32_t)__builtin_rintf(a * 512.0f);
  uint32_t code = a < 0.015625f ? sub : nrm;
  code = a >= 448.0f ? 0x7Eu : code;
  return sign | code;
}

// floor(log2 a) of a finite a > 0 (binary32, subnormals included).
__device__ __forceinline__ int floor_log2(float a) {
  const uint32_t u = __float_as_uint(a);
  const int e = (int)(u >> 23);
  if (e) return e - 127;
  return -127 - __clz(u << 9);  // subnormal: the leading one of the mantissa
}

// The E8M0 code and the unit 2^-shared of a block with largest magnitude
// amax: shared = floor(log2 amax) - 8 clamped to [-127, 127] (-127 for an
// all-zero block).
__device__ __forceinline__ uint32_t mxfp8_scale(float amax, int* neg_shared) {
  int sh = amax > 0.0f ? floor_log2(amax) - 8 : -127;
  sh = sh < -127 ? -127 : (sh > 127 ? 127 : sh);
  *neg_shared = -sh;
  return (uint32_t)(sh + 127);
}

// Four codes of v[0..3] packed lowest first: CDNA4's OCP FP8 conversion
// (round to nearest even, subnormals included) on values clamped to
// [-448, 448] first, since it would turn a larger magnitude into NaN rather
// than saturate; bit-identical to e4m3_encode_rne (checked against the
// oracle's quantiser through moe_quantize_mxfp8).
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  typedef short s16x2_t __attribute__((ext_vector_type(2)));
  const float m = 448.0f;
  s16x2_t w = {0, 0};
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, __builtin_amdgcn_fmed3f(a, -m, m), __builtin_amdgcn_fmed3f(b, -m, m),
                                               1.0f, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, __builtin_amdgcn_fmed3f(c, -m, m), __builtin_amdgcn_fmed3f(d, -m, m),
                                               1.0f, true);
  return __builtin_bit_cast(uint32_t, w);
}

// 32 values of one block -> 32 codes (8 words) and the scale code.
__device__ __forceinline__ uint32_t quantize_block32(const float (&v)[32], uint32_t (&w)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int ns;
  const uint32_t code = mxfp8_scale(amax, &ns);
#pragma unroll
  for (int q = 0; q < 8; ++q)
    w[q] = pack_e4m3x4(__builtin_ldexpf(v[4 * q], ns), __builtin_ldexpf(v[4 * q + 1], ns),
                       __builtin_ldexpf(v[4 * q + 2], ns), __builtin_ldexpf(v[4 * q + 3], ns));
  return code;
}

// ---------------------------------------------------------------------------
// Activation quantisation: one thread per (row, 32-value block); a wave
// takes 8 rows x 8 consecutive blocks, so its loads are 512-byte row pieces
// and its scale bytes 8 consecutive rows of each block row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quantize_act_mxfp8_kernel(const uint16_t* __restrict__ x, int T, int W,
                                                                 uint8_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales, long ld_s) {
  const int nb = W / kMxBlock, nb8 = ceil_div(nb, 8);
  const long grp = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (grp >= (long)ceil_div(T, 8) * nb8) return;
  const int tg = (int)(grp / nb8), jb = (int)(grp - (long)tg * nb8);
  const int t = tg * 8 + (lane >> 3), j = jb * 8 + (lane & 7);
  if (t >= T || j >= nb) return;
  const uint16_t* src = x + (long)t * W + j * kMxBlock;
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 u = *(const uint4*)(src + 8 * q);
    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * q + 2 * i] = bf16_to_f32(w4[i] & 0xffffu);
      v[8 * q + 2 * i + 1] = bf16_to_f32(w4[i] >> 16);
    }
  }
  uint32_t w[8];
  const uint32_t sc = quantize_block32(v, w);
  uint8_t* dst = codes + (long)t * W + j * kMxBlock;
  *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
  *(uint4*)(dst + 16) = make_uint4(w[4], w[5], w[6], w[7]);
  scales[(long)j * ld_s + t] = (uint8_t)sc;
}

hipError_t launch_quantize_act_mxfp8(const uint16_t* x, int T, int W, uint8_t* codes, uint8_t* scales, long ld_s,
                                     hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (W % kMxBlock || !scales) return hipErrorInvalidValue;
  const long threads = (long)ceil_div(T, 8) * ceil_div(W / kMxBlock, 8) * 64;
  hipLaunchKernelGGL(quantize_act_mxfp8_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, x, T, W,
                     codes, scales, ld_s);
  return hipGetLastError();
}

// Token-order scales -> packed-row order: packed[j][p] = tok[j][route_src[p]
// / K] for the *n_rows packed rows (a device count: the accepted rows of a
// capacity-bounded dispatch).  One thread per (block row j, packed row p).
__global__ __launch_bounds__(256) void gather_mx_scales_kernel(const uint8_t* __restrict__ tok, long ld_t,
                                                               const int32_t* __restrict__ route_src,
                                                               const int32_t* __restrict__ n_rows, int K,
                                                               int nb, int R, uint8_t* __restrict__ packed,
                                                               long ld_r) {
  const long id = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (long)nb * R) return;
  const int j = (int)(id / R), p = (int)(id - (long)j * R);
  if (p >= *n_rows) return;
  packed[(long)j * ld_r + p] = tok[(long)j * ld_t + route_src[p] / K];
}

hipError_t launch_gather_mx_scales(const uint8_t* tok, long ld_t, const int32_t* route_src, const int32_t* n_rows,
                                   int K, int W, int R, uint8_t* packed, long ld_r, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (W % kMxBlock) return hipErrorInvalidValue;
  const long n = (long)(W / kMxBlock) * R;
  hipLaunchKernelGGL(gather_mx_scales_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, tok, ld_t,
                     route_src, n_rows, K, W / kMxBlock, R, packed, ld_r);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The MX grouped GEMM
// ---------------------------------------------------------------------------
namespace {
struct MxLoop {
  uint32_t aoff[2], ac16[2];  // A code loads: row offset + chunk, and the chunk's byte offset
  uint32_t boff;              // B code load: byte offset of the lane's row piece at step 0
  uint32_t btile, bstep2;     // B: the tile's packed block, bytes of one packed 32-column step
  uint32_t nrow;              // B: the lane's tile row (clamped)
  uint32_t ash;               // A scales: the window's offset of the wave's first row (0..3)
  uint32_t asrc;              // A scales: byte offset of the lane's dword in a block row
  uint32_t bsrc;              // B scales: byte offset of the lane's dword in a block row
  uint32_t ard[2];            // A fragment: LDS offsets of chunks 2h, 2h+1 (m block 0)
  uint32_t brd;               // B fragment: LDS offset (n block 0)
};
}  // namespace

template <int MB, int NB>
__device__ __forceinline__ void mx_loop(const Tile& t, const MxLoop& L, const char* Ab, const char* Bb,
                                        char* smem, int wave, int lane, f32x16_t (&acc)[4][2]) {
  const int Kd = t.Kd;
  const int nst = ceil_div(Kd, kMxBK);
  const int nblk = Kd / kMxBlock;
  const uint32_t smem_lds = lds_addr(smem);
  const long ldas = t.ld_as;
  const int N = t.N;
  // load q (0 .. kMxLoads-1) of step st
  auto issue_load = [&](int st, int q) {
    const uint32_t buf = smem_lds + (uint32_t)((st % kMxStages) * kMxStageBytes);
    const uint32_t sbuf = buf + (uint32_t)(kMxAStage + kMxBStage + wave * kMxSWave);
    const int k0 = st * kMxBK;
    if (q < 2) {
      // A codes; on a ragged last step the chunk stays inside the row (its
      // k half is zeroed in the fragment)
      uint32_t off = L.aoff[q] + (uint32_t)k0;
      if (k0 + kMxBK > Kd) off = L.aoff[q] - L.ac16[q] + (uint32_t)min(k0 + (int)L.ac16[q], Kd - 16);
      lds_dma16(Ab, off, buf + (uint32_t)((wave * 2 + q) * 1024));
    } else if (q < 4) {
      // A scales of block 2 st + (q - 2) (the last block again past Kd)
      const int j = min(2 * st + (q - 2), nblk - 1);
      lds_dma4(t.as, (uint32_t)((long)j * ldas) + L.asrc, sbuf + (uint32_t)((q - 2) * 256));
    } else if (q == 4) {
      // B codes: the lane's row piece of packed step 2 st + half (half 1 of
      // a ragged last step reads half 0)
      const int s32 = min(2 * st + (int)(L.boff & 1u), nblk - 1);
      lds_dma16(Bb, L.btile + (uint32_t)s32 * L.bstep2 + L.nrow * 16u, buf + (uint32_t)(kMxAStage + wave * 1024));
    } else {
      // B scales: lanes 0-15 block 2 st, lanes 16-31 block 2 st + 1, the
      // rest block 2 st again (unused)
      const int j = min(2 * st + ((lane >> 4) == 1 ? 1 : 0), nblk - 1);
      lds_dma4(t.e8, (uint32_t)(j * N) + L.bsrc, sbuf + 512u);
    }
  };

  const int h = lane >> 5;
  i32x8_t fa[MB];                          // A fragments (of the step being multiplied)
  uint32_t sa[MB];
  i32x8_t fb[NB > 0 ? NB : 1], fbn[NB > 0 ? NB : 1];  // B fragments of this step and the next
  uint32_t sb[NB > 0 ? NB : 1], sbn[NB > 0 ? NB : 1];
  auto stage_of = [&](int st) { return smem + (st % kMxStages) * kMxStageBytes; };
  auto read_a = [&](int st, int mb, bool half_valid) {
    const char* stg = stage_of(st);
    const uint4 lo = *(const uint4*)(stg + L.ard[0] + mb * 32 * kMxARow);
    uint4 hi = *(const uint4*)(stg + L.ard[1] + mb * 32 * kMxARow);
    // a ragged last step has no K block 1: its codes (bytes 16-31 of every
    // lane) are zeroed
    if (!half_valid) hi = make_uint4(0, 0, 0, 0);
    fa[mb] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    const char* sw = stg + kMxAStage + kMxBStage + wave * kMxSWave;
    sa[mb] = *(const uint8_t*)(sw + h * 256 + L.ash + mb * 32 + (lane & 31));
  };
  auto read_b = [&](int st, i32x8_t (&b)[NB > 0 ? NB : 1], uint32_t (&s)[NB > 0 ? NB : 1]) {
    const char* stg = stage_of(st);
    const char* sw = stg + kMxAStage + kMxBStage + wave * kMxSWave;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint4 q = *(const uint4*)(stg + kMxAStage + L.brd + nb * 32 * kMxBRow);
      b[nb] = i32x8_t{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
      s[nb] = *(const uint8_t*)(sw + 512 + h * 64 + nb * 32 + (lane & 31));
    }
  };
  // wait until step st's loads have landed, with `later` steps issued after
  // it still in flight; every wave's reads of earlier stages are complete
  // (lgkmcnt) before the barrier, so a stage may be refilled after it
  auto wait_landed = [&](int later) {
    if (later >= 3)
      wait_vmcnt<3 * kMxLoads>();
    else if (later == 2)
      wait_vmcnt<2 * kMxLoads>();
    else if (later == 1)
      wait_vmcnt<kMxLoads>();
    else
      wait_vmcnt<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  // steps 0 .. kMxStages - 2 in flight before the loop
  for (int st = 0; st < kMxStages - 1; ++st)
    if (st < nst)
#pragma unroll
      for (int q = 0; q < kMxLoads; ++q) issue_load(st, q);
  wait_landed(min(nst - 1, kMxStages - 2));
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) read_a(0, mb, Kd >= kMxBK);
  read_b(0, fb, sb);
  // Step kt: wait for step kt + 1 and pass the barrier, refill the stage of
  // step kt - 1 with step kt + 4, then issue step kt's MFMAs, each m block's
  // followed by the reads of that block's next-step fragments, so LDS reads
  // run under the MFMAs
  for (int kt = 0; kt < nst; ++kt) {
    const bool more = kt + 1 < nst;
    if (more) {
      wait_landed(min(nst - 1, kt + kMxStages - 2) - (kt + 1));
      const int nxt = kt + kMxStages - 1;
      if (nxt < nst)
#pragma unroll
        for (int q = 0; q < kMxLoads; ++q) issue_load(nxt, q);
      read_b(kt + 1, fbn, sbn);
    }
    const bool half_next = Kd >= (kt + 2) * kMxBK;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma_mx(fa[mb], fb[nb], sa[mb], sb[nb], acc[mb][nb]);
      if (more) read_a(kt + 1, mb, half_next);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      fb[nb] = fbn[nb];
      sb[nb] = sbn[nb];
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(kMxThreads, 1) void gemm_mx_kernel(GemmArgs a) {
  __shared__ __align__(1024) char smem[kMxSmem];
  Tile t;
  if (!decode_tile(a, t, kChunkRows, kTileN)) return;
  const char* Ab = (const char*)t.A;
  const char* Bb = (const char*)t.B;
  if (t.g > 0) Bb += (long)(t.g - 1) * a.strideB / 2;  // MXFP4: half a byte per element

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave_m = wave / kMxWaveN, wave_n = wave % kMxWaveN;

  // the tile's 32-row blocks split evenly between the two wave rows
  const int mblk = ceil_div(min(t.mcount, kChunkRows), 32);
  const int msplit = (mblk + 1) >> 1;
  const int row0 = wave_m * msplit * 32;
  const int mbn = wave_m == 0 ? msplit : mblk - msplit;
  const int ncols = t.N - (t.n0 + wave_n * 64);
  const int nbn = mbn == 0 ? 0 : (ncols >= 64 ? 2 : (ncols > 0 ? ceil_div(ncols, 32) : 0));

  MxLoop L;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int r = (wave * 2 + s) * 16 + (lane >> 2);
    L.ac16[s] = (uint32_t)(((lane & 3) ^ swz_rows(r)) * 16);
    L.aoff[s] = (uint32_t)(src_row(t, r) * t.lda) + L.ac16[s];
  }
  {
    const int rn = min(kTileN, t.N - t.n0);  // rows of the packed tile
    L.btile = (uint32_t)((long)t.n0 * t.Kd / 2);
    L.bstep2 = (uint32_t)(rn * 16);
    const int gl = wave * 64 + lane;
    const int n = gl >> 1;
    const int half = (gl & 1) ^ ((n >> 3) & 1);
    L.nrow = (uint32_t)min(n, rn - 1);
    L.boff = (uint32_t)half;  // the packed step's parity (the half this lane loads)
  }
  {
    // scale row of the wave's first row; a wave with no rows past the
    // matrix's last row reads a window inside it (ld_as has 256 bytes of
    // slack past the rows, so the 256-byte window of a real row stays in
    // its block row)
    const long g0 = min(t.rowbase + t.m0 + row0, t.ld_as - 256);
    L.ash = (uint32_t)(g0 & 3);
    L.asrc = (uint32_t)((g0 & ~3L) + 4 * lane);
    const int c0 = min(t.n0 + wave_n * 64 + 4 * (lane & 15), t.N - 4);
    L.bsrc = (uint32_t)c0;
  }
  {
    const int r = lane & 31, h = lane >> 5;
    const int rr = row0 + r;
    L.ard[0] = (uint32_t)(rr * kMxARow + ((h ^ swz_rows(rr)) << 4));
    L.ard[1] = (uint32_t)(rr * kMxARow + (((2 + h) ^ swz_rows(rr)) << 4));
    const int n = wave_n * 64 + r;
    L.brd = (uint32_t)(n * kMxBRow + ((h ^ ((n >> 3) & 1)) << 4));
  }

  f32x16_t acc[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

#define MOE_MXLOOP(MB_, NB_) mx_loop<MB_, NB_>(t, L, Ab, Bb, smem, wave, lane, acc)
  switch (nbn * 4 + (max(mbn, 1) - 1)) {
    case 0: case 1: case 2: case 3:
      // no columns for this wave: it still issues its share of every load
      MOE_MXLOOP(1, 0); break;
    case 4: MOE_MXLOOP(1, 1); break;
    case 5: MOE_MXLOOP(2, 1); break;
    case 6: MOE_MXLOOP(3, 1); break;
    case 7: MOE_MXLOOP(4, 1); break;
    case 8: MOE_MXLOOP(1, 2); break;
    case 9: MOE_MXLOOP(2, 2); break;
    case 10: MOE_MXLOOP(3, 2); break;
    default: MOE_MXLOOP(4, 2); break;
  }
#undef MOE_MXLOOP
  // every wave's loads have landed and been read: the LDS is free
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // accumulator layout of the 32x32 MFMA: lane l, register r holds row
  // 8*(r/4) + 4*(l/32) + r%4, column l%32, of the wave's rows from row0
  if constexpr (EPI == EPI_QRELU2) {
    if (nbn == 0) return;
    float* stage = (float*)(smem + wave * (64 * kMxEpiRow * 4));
    uint8_t* C = (uint8_t*)t.C;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      // rows pass*64 .. +63 of the wave: m blocks 2 pass, 2 pass + 1
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) {
        const int mb = 2 * pass + m2;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int lr = m2 * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const float u = fmaxf(acc[mb][nb][r], 0.0f);
            stage[lr * kMxEpiRow + nb * 32 + (lane & 31)] = u * u;
          }
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // lane -> (row, block): 64 rows x 2 blocks, two per lane
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int lr = lane;          // staged row
        const int blk = it;           // 32-column block of the wave's 64 columns
        const int row = row0 + pass * 64 + lr;
        const int col = t.n0 + wave_n * 64 + blk * 32;
        float v[32];
        const float* src = stage + lr * kMxEpiRow + blk * 32;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float4 f = *(const float4*)(src + 4 * q);
          v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
        }
        if (pass * 64 + lr < mbn * 32 && row < t.mcount && col < t.N) {
          uint32_t w[8];
          const uint32_t sc = quantize_block32(v, w);
          const long orow = t.rowbase + t.m0 + row;
          uint8_t* dst = C + orow * t.ldc + col;
          *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
          *(uint4*)(dst + 16) = make_uint4(w[4], w[5], w[6], w[7]);
          t.cs[(long)(col / kMxBlock) * t.ld_cs + orow] = (uint8_t)sc;
        }
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    return;
  } else {
    if (t.cf32) {
      if (nbn == 0) return;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb >= mbn) continue;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          if (nb >= nbn) continue;
          const int col = t.n0 + wave_n * 64 + nb * 32 + (lane & 31);
          if (col >= t.N) continue;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = row0 + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row < t.mcount) ((float*)t.C)[(t.rowbase + t.m0 + row) * t.ldc + col] = acc[mb][nb][r];
          }
        }
      }
      return;
    }
    if (nbn == 0) return;
    uint16_t* stage = (uint16_t*)(smem + wave * (128 * 64 * 2));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if (mb >= mbn) continue;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int lc = nb * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          stage[lr * 64 + lc] = (uint16_t)f32_to_bf16(acc[mb][nb][r]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    uint16_t* C = (uint16_t*)t.C;
#pragma unroll 4
    for (int it = 0; it < 128 * 8 / 64; ++it) {
      const int id = it * 64 + lane;
      const int lr = id >> 3, c = id & 7;
      const int col = t.n0 + wave_n * 64 + c * 8;
      if (lr < mbn * 32 && row0 + lr < t.mcount && col < t.N) {
        const uint4 v = *(const uint4*)(stage + lr * 64 + c * 8);
        *(uint4*)(C + (t.rowbase + t.m0 + row0 + lr) * t.ldc + col) = v;
      }
    }
  }
}

hipError_t launch_gemm_mx(const GemmArgs& a, int epi, int max_tiles, hipStream_t s) {
  if (!a.plan || max_tiles <= 0) return max_tiles <= 0 ? hipSuccess : hipErrorInvalidValue;
  if (a.Kd % kMxBlock || a.N % kMxBlock || (a.M_s > 0 && (a.Kd_s % kMxBlock || a.N_s % kMxBlock)))
    return hipErrorInvalidValue;
  if (a.ld_as % 4 || (a.M_s > 0 && a.ld_as_s % 4)) return hipErrorInvalidValue;
  const dim3 grid(xcd_grid(max_tiles)), block(kMxThreads);
  if (epi == EPI_QRELU2)
    hipLaunchKernelGGL(gemm_mx_kernel<EPI_QRELU2>, grid, block, 0, s, a);
  else if (epi == EPI_STORE)
    hipLaunchKernelGGL(gemm_mx_kernel<EPI_STORE>, grid, block, 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe
