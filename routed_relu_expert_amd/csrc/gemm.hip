// Grouped GEMMs of the routed experts, the shared expert and the dense
// projections (router in bf16x3 form, latent in/out).
//
// Main bf16 kernel (gemm_bf16_mfma_kernel): v_mfma_f32_32x32x16_bf16 on
// CDNA4.  A workgroup of 8 waves (2 x 4) computes a 256-row x 256-column
// tile, each wave 128 x 64 (4 x 2 MFMA blocks of 32 x 32); the tile's 32-row
// blocks are split evenly between the two wave rows, so a partly filled row
// chunk (the tail of an expert's rows) leaves no wave idle.  K runs in steps
// of 32 through a ring of LDS stages (4 stages of 32 KB; 5 of 24 KB when B
// is FP8) filled by direct global->LDS loads (global_load_lds_dwordx4)
// issued one step less than the ring ahead (3 steps, 4 with FP8 B) and
// spread over the two k16 sub-steps, tracked
// with explicit vmcnt waits; one barrier per step.  Rows of the A operand are
// gathered through the route map on the fly, so the packed [R, d] input is
// never materialised.  B comes from the packed weight layout (one contiguous
// block per tile and K step).
//
// LDS layouts (16-byte chunks, XOR-swizzled so the fragment reads are free
// of bank conflicts):
//  * K-contiguous tiles (A, and bf16 B stored [N][K]): 64 bytes per row,
//    chunk c of row r at position c ^ ((r >> 2) & 3).  Fragments are read
//    with ds_read_b128.
//  * bf16 B stored [K][N] (the neuron-major down projections): 2*256 bytes
//    per k row, chunk c of k row k at position c ^ S[k & 3], S = {0, 4, 10,
//    14}.  Fragments are read with the CDNA4 transpose load
//    ds_read_b64_tr_b16: in each group of 16 lanes, source lane 4q + r points
//    at k row q and columns 4r..4r+3, and output lane i receives rows 0..3 of
//    column i, so two transpose loads give a lane the 8 consecutive k of its
//    column that the MFMA B operand needs.
//  * FP8 B (E4M3 codes; W8A16): [N][K] rows of 32 bytes, chunk h of row r at
//    position h ^ ((r >> 3) & 1), read 8 bytes per lane; [K][N] rows of 256
//    bytes, chunk c of k row k at position c ^ (2 (k & 7)), read with
//    ds_read_b64_tr_b8 (in each group of 16 lanes, source lane 2q + h points
//    at k row q, bytes 8h..8h+7, and output lane i receives rows 0..7 of
//    column i).  The codes are widened to bf16 in registers (exact) and the
//    output column's fp32 scale multiplies the fp32 sum in the epilogue.
//  * MXFP4 B (E2M1 codes, W4A16; [N][K] only): rows of 16 bytes per K step
//    (32 codes, one scale block), 4-byte word w of row r at position
//    w ^ ((r >> 3) & 3), read 4 bytes (8 codes) per lane; each wave also
//    keeps its own copy of the step's 256 E8M0 scales (one per tile row).
//    Codes are widened to bf16 times their block scale in registers (exact),
//    so the MFMA sums the dequantised weights.
// The epilogue goes through LDS for bf16 outputs so every global store is a
// 16-byte row segment.
//
// Split-K dense kernel (gemm_bf16_splitk_kernel, the router's bf16x3 GEMM):
// 128 x 128 tiles, register-staged LDS, split-K partials.
// fp32 kernel (the tiny fp32 layer): the same plan tiles with plain fp32
// FMAs.
//
// Epilogues: ReLU^2 with the rounding points bf16(relu(bf16(u))^2) of the
// NemotronH "Arithmetic" section (plain relu(u)^2 in fp32); plain store
// (bf16 or fp32); add an fp32 addend (and optionally the old output) before
// the single rounding.
#include "moe_internal.h"
#include "tile.h"

#include <type_traits>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma_32x32x16(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Epilogue value of one output element (before the final rounding of bf16
// outputs; fp32 outputs store it as is).
template <int EPI>
__device__ __forceinline__ float epilogue_value(const GemmArgs& a, const Tile& t, long orow, int col,
                                                float v) {
  if (EPI == EPI_RELU2) {
    if (t.cf32) {
      const float r = fmaxf(v, 0.0f);
      return r * r;
    }
    const float r = fmaxf(bf16_round(v), 0.0f);
    return r * r;
  }
  if (EPI == EPI_DRELU2) {
    const float h = bf16_to_f32(((const uint16_t*)t.aux)[orow * t.ldc + col]);
    return v * (2.0f * sqrtf(h));
  }
  if (EPI == EPI_ADD_F32) {
    if (a.addend) v += a.addend[orow * a.ld_add + col];
    if (a.resid)
      v += t.cf32 ? ((const float*)a.resid)[orow * t.ldc + col]
                  : bf16_to_f32(((const uint16_t*)a.resid)[orow * t.ldc + col]);
  }
  return v;
}

// NT: a streaming store, for the large fp32 outputs written once and not
// read again by the launch: the weight gradients and the [K][N]-B products'
// fp32 rows (the backward's recomputed U and its dx rows)
template <int EPI, bool NT = false>
__device__ __forceinline__ void epilogue_store(const GemmArgs& a, const Tile& t, int row, int col,
                                               float v) {
  const long orow = t.rowbase + t.m0 + row;
  v = epilogue_value<EPI>(a, t, orow, col, v);
  if (NT)
    __builtin_nontemporal_store(v, (float*)t.C + orow * t.ldc + col);
  else if (t.cf32)
    ((float*)t.C)[orow * t.ldc + col] = v;
  else
    ((uint16_t*)t.C)[orow * t.ldc + col] = (uint16_t)f32_to_bf16(v);
}

// ---------------------------------------------------------------------------
// Main bf16 MFMA kernel: 256 x 256 tiles, 4-stage direct-to-LDS pipeline
// ---------------------------------------------------------------------------
namespace {
constexpr int kWaveM = 2, kWaveN = 4;            // wave grid; each wave owns 128 x 64
constexpr int kWaves = kWaveM * kWaveN;
constexpr int kThreads = kWaves * 64;
constexpr int kBK = 32;                          // K per pipeline step
constexpr int kRowBytes = kBK * 2;               // 64-byte A tile rows (4 chunks)
constexpr int kAStage = kChunkRows * kRowBytes;  // 16 KB
constexpr int kLoadsA = kAStage / 1024 / kWaves; // 1 KB segments per wave per step
constexpr int kSub = kBK / 16;                   // k16 MFMA sub-steps per step
// The B operand (WF): bf16 (0), FP8 codes (1, half the bytes: a fifth ring
// stage fits in the LDS the epilogue needs anyway) or MXFP4 codes (2: 4 KB
// of codes and 8 per-wave copies of the step's 256 scale bytes).
template <int WF>
struct Pipe {
  static constexpr bool W8 = WF == 1, W4 = WF == 2;
  static constexpr int kEB = W8 ? 1 : 2;              // bytes per B element (bf16, FP8)
  static constexpr int kEB2 = W4 ? 1 : 2 * kEB;       // bytes per 2 B elements
  static constexpr int kBRowBytes = kBK * kEB2 / 2;   // B_NK: a tile row of one step
  static constexpr int kBKRowBytes = kTileN * kEB;    // B_KN: one k row of the tile
  static constexpr int kBCodes = kTileN * kBRowBytes; // 16 KB / 8 KB / 4 KB of codes per step
  static constexpr int kBStage = kBCodes + (W4 ? kWaves * kTileN : 0);
  static constexpr int kStageBytes = kAStage + kBStage;
  static constexpr int kStages = (W8 || W4) ? 5 : 4;
  // 1 KB loads of B per wave and step; MXFP4: two 256-byte code loads and
  // one 256-byte scale load
  static constexpr int kLoadsB = W4 ? 3 : kBStage / 1024 / kWaves;
  static constexpr int kLoads = kLoadsA + kLoadsB;    // 1 KB loads per wave per step
  static constexpr int kRing = kStages * kStageBytes;
  static constexpr int kEpi = kWaves * 128 * 64 * 2;  // the epilogue's bf16 staging
  static constexpr int kSmem = kRing > kEpi ? kRing : kEpi;
  static_assert(kStages >= 2 && kStages <= 5, "the vmcnt waits cover at most 3 later steps in flight");
  static_assert(kSmem <= 160 * 1024, "fits the LDS of a CU");
};
static_assert(kWaveM * 128 == kChunkRows && kWaveN * 64 == kTileN, "wave grid covers the tile");
static_assert(kTileN == kPackTile && kBK == kPackStep, "a tile reads whole blocks of the packed weights");
}  // namespace

template <int WF>
struct MainLoop {
  static constexpr int kLoadsB = Pipe<WF>::kLoadsB;
  // per-lane byte offsets of the loads at k = 0, relative to the A / B base
  // pointers, and the lane's chunk offset within a K step
  uint32_t aoff[kLoadsA], ac16[kLoadsA];
  uint32_t boff[kLoadsB], bc16[kLoadsB];
  int kb_row[kLoadsB];  // B_NK: tile row of each load; B_KN: k row within the step
  // packed B: byte offset of the tile's block and the bytes one K step
  // (B_NK) or one k row (B_KN) of the tile takes
  uint32_t btile, bstep;
  // per-lane LDS read offsets, relative to the stage's A / B region
  uint32_t ard[kSub];     // A fragment of k16 sub-step kk, m block 0 (block mb adds 32 rows)
  uint32_t brd_nk[kSub];  // B stored [N][K]: fragment of sub-step kk, n block 0 (+32 rows per nb)
  uint32_t brd_kn[2];     // B stored [K][N]: transpose-load address of n block nb, k16 step 0
  uint32_t srd;           // MXFP4: the lane's column in its wave's copy of the step's scales (n block 0)
};

// The k order inside a K step.  bf16 B: sub-step kk, lane half h (lanes
// 32h .. 32h+31) takes k = 16 kk + 8 h .. +7 (A chunk 2 kk + h).  FP8 B: the
// same lanes take k = 16 h + 8 kk .. +7 (A chunk 2 h + kk), so a lane's two
// sub-steps read one 16-byte range of a B_NK row; the dot product is the same
// sum over the step's 32 k.
template <int WF>
__device__ __forceinline__ int a_chunk(int kk, int lane) {
  return WF == 1 ? (lane >> 5) * 2 + kk : kk * 2 + (lane >> 5);
}

template <int BMODE, int MB, int NB, int WF, bool SPLIT>
__device__ __forceinline__ void mfma_loop(const Tile& t, const MainLoop<WF>& L, const char* Abase,
                                          const char* Bbase, const char* Sbase, char* smem, int wave, int row0,
                                          int lane, f32x16_t (&acc)[4][2]) {
  using P = Pipe<WF>;
  constexpr bool W8 = P::W8, W4 = P::W4;
  static_assert(!W4 || BMODE == B_NK, "MXFP4 B is read from [N][K] tiles");
  constexpr int kStages = P::kStages, kStageBytes = P::kStageBytes, kLoadsB = P::kLoadsB;
  // K steps [st_begin, st_end): the whole K, or (SPLIT) a split's share of
  // it (decode_tile gives the range in 64-wide units)
  const int st_begin = SPLIT ? 2 * t.k_begin : 0;
  const int st_end = SPLIT ? min(2 * t.k_end, ceil_div(t.Kd, kBK)) : ceil_div(t.Kd, kBK);
  const int Kd = t.Kd;
  const uint32_t smem_lds = lds_addr(smem);
  // Load q (0 .. kLoads-1) of step st: A segments first, then B segments.
  // chk: whether step st may be the ragged last one (steady-state steps pass
  // std::false_type, so their loads carry no check)
  auto issue_load = [&](int st, int q, auto chk) {
    const uint32_t buf = smem_lds + (uint32_t)((st % kStages) * kStageBytes);
    const int k0 = st * kBK;
    const bool ragged = decltype(chk)::value && k0 + kBK > Kd;
    if (q < kLoadsA) {
      const int s = q;
      uint32_t off = L.aoff[s] + (uint32_t)k0 * 2u;
      if (ragged)  // keep the chunk inside the row: columns >= Kd are zeroed in the A fragment
        off = L.aoff[s] - L.ac16[s] + (uint32_t)min(k0 * 2 + (int)L.ac16[s], (Kd - 8) * 2);
      lds_dma16(Abase, off, buf + (uint32_t)((wave * kLoadsA + s) * 1024));
    } else if constexpr (W4) {
      // codes: two 256-byte segments (16 tile rows each) per wave; scales:
      // the step's row of the block-major scale matrix, into the wave's copy
      const int s = q - kLoadsA;
      if (s < 2)
        lds_dma4(Bbase, L.boff[s] + (uint32_t)st * L.bstep,
                 buf + (uint32_t)(kAStage + (wave * 2 + s) * 256));
      else
        lds_dma4(Sbase, L.boff[2] + (uint32_t)st * (uint32_t)t.N,
                 buf + (uint32_t)(kAStage + P::kBCodes + wave * 256));
    } else {
      const int s = q - kLoadsA;
      uint32_t off;
      if (BMODE == B_NKP) {
        // plain rows: like A, the chunk stays inside the row on a ragged step
        off = L.boff[s] + (uint32_t)k0 * 2u;
        if (ragged) off = L.boff[s] - L.bc16[s] + (uint32_t)min(k0 * 2 + (int)L.bc16[s], (Kd - 8) * 2);
      } else if (BMODE == B_NK) {
        // packed: step st of the tile is a [rn][32] block (ragged: [rn][Kd - k0])
        off = L.boff[s] + (uint32_t)st * L.bstep;
        if (ragged) {
          const int kwb = (Kd - k0) * P::kEB;
          off = L.btile + (uint32_t)st * L.bstep + (uint32_t)(L.kb_row[s] * kwb) +
                (uint32_t)min((int)L.bc16[s], kwb - 16);
        }
      } else {
        // packed: the tile's column strip is row-major [Kd][cn]
        const int kr = min(k0 + L.kb_row[s], Kd - 1);
        off = L.boff[s] + (uint32_t)kr * L.bstep;
      }
      lds_dma16(Bbase, off, buf + (uint32_t)(kAStage + (wave * kLoadsB + s) * 1024));
    }
  };
  auto issue_one = [&](int st, int q) { issue_load(st, q, std::true_type{}); };
  constexpr int kLoads = P::kLoads;

  struct Frags {
    uint4 a[MB];
    uint4 b[NB > 0 ? NB : 1];
  };
  auto read_frags = [&](const char* sa, const char* sb, int kk, int kvalid, Frags& f) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) f.a[mb] = *(const uint4*)(sa + L.ard[kk] + mb * 32 * kRowBytes);
    if (kvalid < kBK) {
      if (a_chunk<WF>(kk, lane) * 8 >= kvalid)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) f.a[mb] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (W4) {
        // 8 codes of the lane's column and k half, times the column's scale
        const uint32_t wd = *(const uint32_t*)(sb + L.brd_nk[kk] + nb * 32 * P::kBRowBytes);
        const float sc = e8m0_to_f32(*(const uint8_t*)(sb + P::kBCodes + L.srd + nb * 32));
        f.b[nb] = fp4x8_to_bf16x8(wd, sc);
      } else if (BMODE != B_KN) {
        if (W8)
          f.b[nb] = fp8x8_to_bf16x8(*(const uint2*)(sb + L.brd_nk[kk] + nb * 32 * P::kBRowBytes));
        else
          f.b[nb] = *(const uint4*)(sb + L.brd_nk[kk] + nb * 32 * P::kBRowBytes);
      } else if (W8) {
        // sub-step kk is 8 k rows further; one 8-bit transpose load gives
        // the lane the 8 k of its column
        const char* p = sb + L.brd_kn[nb] + kk * (8 * P::kBKRowBytes);
        const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)p);
        f.b[nb] = fp8x8_to_bf16x8(__builtin_bit_cast(uint2, v));
      } else {
        // k16 step kk is 16 k rows further: +kk * 16 * 512 bytes; the high
        // half (k + 4) is 4 rows further; the swizzle repeats every 4 rows
        const char* p = sb + L.brd_kn[nb] + kk * (16 * P::kBKRowBytes);
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 4 * P::kBKRowBytes));
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        f.b[nb] = make_uint4(l2.x, l2.y, h2.x, h2.y);
      }
    }
  };

  // Wait until step st's loads have landed (the loads of the steps issued
  // after it may stay in flight), then a barrier makes every wave's part
  // of the step visible.
  auto wait_step = [&](int st) {
    const int later = min(st_end - 1, st + kStages - 2) - st;  // steps issued after st
    if (later >= 3)
      wait_vmcnt<3 * kLoads>();
    else if (later == 2)
      wait_vmcnt<2 * kLoads>();
    else if (later == 1)
      wait_vmcnt<kLoads>();
    else
      wait_vmcnt<0>();
    asm volatile("s_barrier" ::: "memory");
  };
  auto stage_a = [&](int st) { return smem + (st % kStages) * kStageBytes + row0 * kRowBytes; };
  auto stage_b = [&](int st) { return smem + (st % kStages) * kStageBytes + kAStage; };

  // Steps st_begin .. st_begin + kStages-2 are in flight before the loop.  During step kt the
  // loads of step kt + kStages - 1 are issued (into the buffer of step
  // kt - 1, which every wave finished reading before the last barrier), and
  // after the MFMAs of its last k16 sub-step are issued the wave waits for
  // step kt + 1 and reads its first fragments, so that LDS latency overlaps
  // the tail of step kt's MFMAs.
#pragma unroll
  for (int st = 0; st < kStages - 1; ++st)
    if (st_begin + st < st_end)
#pragma unroll
      for (int q = 0; q < kLoads; ++q) issue_one(st_begin + st, q);
  wait_step(st_begin);
  Frags cur, nxt;
  if (NB > 0) read_frags(stage_a(st_begin), stage_b(st_begin), 0, Kd - st_begin * kBK, cur);
  // One K step.  STEADY (a std::integral_constant): steps whose loads,
  // wait and fragments are all full-width and not the last -- kt <
  // st_end - kStages -- so the next loads are always issued, none can be
  // ragged and the wait keeps kStages - 2 later steps in flight; the last
  // steps take the general form.
  auto step = [&](int kt, auto steady) {
    constexpr bool kSteady = decltype(steady)::value;
    const int nxt_st = kt + kStages - 1;
    const bool more = kSteady || nxt_st < st_end;
    const char* sa = stage_a(kt);
    const char* sb = stage_b(kt);
    const int kvalid = kSteady ? 2 * kBK : Kd - kt * kBK;  // < kBK only on a ragged last step
#pragma unroll
    for (int kk = 0; kk < kSub; ++kk) {
      if (more)
#pragma unroll
        for (int q = kk * kLoads / kSub; q < (kk + 1) * kLoads / kSub; ++q)
          issue_load(nxt_st, q, std::integral_constant<bool, !kSteady>{});
      if (kk + 1 < kSub) {
        if (NB > 0) {
          read_frags(sa, sb, kk + 1, kvalid, nxt);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma_32x32x16(cur.a[mb], cur.b[nb], acc[mb][nb]);
          cur = nxt;
        }
      } else {
        if (NB > 0)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma_32x32x16(cur.a[mb], cur.b[nb], acc[mb][nb]);
        if (kSteady || kt + 1 < st_end) {
          if (kSteady) {
            static_assert(kStages - 2 <= 3, "the vmcnt waits cover at most 3 later steps in flight");
            wait_vmcnt<(kStages - 2) * kLoads>();
            asm volatile("s_barrier" ::: "memory");
          } else {
            wait_step(kt + 1);
          }
          if (NB > 0) read_frags(stage_a(kt + 1), stage_b(kt + 1), 0, kvalid - kBK, cur);
        }
      }
    }
  };
  int kt = st_begin;
  for (; kt < st_end - kStages; ++kt) step(kt, std::true_type{});
  for (; kt < st_end; ++kt) step(kt, std::false_type{});
}

template <int BMODE, int EPI, int WF, bool SPLIT = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_mfma_kernel(GemmArgs a) {
  using P = Pipe<WF>;
  constexpr bool W8 = P::W8, W4 = P::W4;
  __shared__ __align__(1024) char smem[P::kSmem];

  Tile t;
  if (!decode_tile(a, t, kChunkRows, kTileN)) return;
  const uint16_t* A = (const uint16_t*)t.A;
  const char* Bb = (const char*)t.B;
  if (t.g > 0) Bb += (long)(t.g - 1) * a.strideB * P::kEB2 / 2;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave_m = wave / kWaveN, wave_n = wave % kWaveN;
  const char* Sb = (const char*)t.e8;

  // ---- per-lane load sources and LDS read offsets ----
  MainLoop<WF> L;
  L.btile = (uint32_t)((long)t.n0 * t.Kd * P::kEB2 / 2);
  {
    const int nrem = min(kTileN, t.N - t.n0);  // rows (B_NK) or columns (B_KN) of the packed tile
    L.bstep = (uint32_t)(BMODE == B_NK ? nrem * P::kBRowBytes : nrem * P::kEB);
  }
#pragma unroll
  for (int s = 0; s < kLoadsA; ++s) {
    // segment wave*kLoadsA + s holds rows seg*16 .. seg*16+15, 4 chunks each
    const int r = (wave * kLoadsA + s) * 16 + (lane >> 2);
    L.ac16[s] = (uint32_t)(((lane & 3) ^ swz_rows(r)) * 16);
    L.aoff[s] = (uint32_t)(src_row(t, r) * t.lda * 2) + L.ac16[s];
  }
#pragma unroll
  for (int s = 0; s < P::kLoadsB; ++s) {
    const int seg = wave * P::kLoadsB + s;
    if (W4) {
      if (s < 2) {
        // segment wave*2 + s: tile rows 16 (wave*2 + s) .. +15; lane i fills
        // LDS word i % 4 of row i / 4, which holds the row's word
        // (i % 4) ^ ((row >> 3) & 3)
        const int r = (wave * 2 + s) * 16 + (lane >> 2);
        const int rc = min(r, t.N - t.n0 - 1);
        const int wsrc = (lane & 3) ^ ((r >> 3) & 3);
        L.boff[s] = L.btile + (uint32_t)(rc * P::kBRowBytes + wsrc * 4);
      } else {
        // scales of tile columns 4 lane .. +3 (kept inside the matrix row:
        // N - n0 is a multiple of 32)
        L.boff[s] = (uint32_t)(t.n0 + min(4 * lane, t.N - t.n0 - 4));
      }
      L.bc16[s] = 0;
      L.kb_row[s] = 0;
    } else if (BMODE != B_KN) {
      // bf16: 16 rows of 4 chunks per segment; FP8: 32 rows of 2 chunks,
      // chunk h of row r at position h ^ ((r >> 3) & 1)
      const int r = W8 ? seg * 32 + (lane >> 1) : seg * 16 + (lane >> 2);
      const int rc = min(r, t.N - t.n0 - 1);  // row inside the packed tile
      L.bc16[s] = (uint32_t)((W8 ? ((lane & 1) ^ ((r >> 3) & 1)) : ((lane & 3) ^ swz_rows(r))) * 16);
      L.kb_row[s] = rc;
      L.boff[s] = BMODE == B_NKP ? (uint32_t)((long)(t.n0 + rc) * t.ldb * 2) + L.bc16[s]
                                 : L.btile + (uint32_t)(rc * P::kBRowBytes) + L.bc16[s];
    } else {
      // bf16: 2 k rows of 32 chunks per segment; FP8: 4 k rows of 16
      // chunks, chunk c of k row k at position c ^ (2 (k & 7))
      int kr, c;
      if (W8) {
        kr = seg * 4 + (lane >> 4);
        c = (lane & 15) ^ (2 * (kr & 7));
      } else {
        kr = seg * 2 + (lane >> 5);
        c = (lane & 31) ^ swz_krow(kr);
      }
      L.kb_row[s] = kr;
      L.bc16[s] = (uint32_t)min(c * 16, (t.N - t.n0) * P::kEB - 16);  // byte offset in the strip row
      L.boff[s] = L.btile + L.bc16[s];
    }
  }
#pragma unroll
  for (int kk = 0; kk < kSub; ++kk) {
    const int r = lane & 31, c = a_chunk<WF>(kk, lane);
    L.ard[kk] = (uint32_t)(r * kRowBytes + ((c ^ swz_rows(r)) << 4));
    if (W4) {
      // word 2 kk + h of tile row n = wave_n * 64 + r (n block 0)
      const int n = wave_n * 64 + r, w = 2 * kk + (lane >> 5);
      L.brd_nk[kk] = (uint32_t)(n * P::kBRowBytes + ((w ^ ((n >> 3) & 3)) << 2));
    } else if (W8) {
      const int h = lane >> 5;
      L.brd_nk[kk] = (uint32_t)((wave_n * 64 + r) * P::kBRowBytes + ((h ^ ((r >> 3) & 1)) << 4) + kk * 8);
    } else {
      L.brd_nk[kk] = (uint32_t)(wave_n * 64 * kRowBytes) + L.ard[kk];
    }
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int g = lane >> 4, j = lane & 15;
    if (W8) {
      // group g of 16 lanes: columns (g & 1) * 16 .. +15 of the n block, k
      // half g >> 1; lane j points at k row j >> 1, bytes 8 (j & 1) .. +7
      const int chunk = wave_n * 4 + nb * 2 + (g & 1);
      const int q = j >> 1;
      const int kr = (g >> 1) * 16 + q;
      L.brd_kn[nb] = (uint32_t)(kr * P::kBKRowBytes + ((chunk ^ (2 * q)) << 4) + (j & 1) * 8);
    } else {
      const int n = wave_n * 64 + nb * 32 + (g & 1) * 16 + 4 * (j & 3);
      const int kr = (g >> 1) * 8 + (j >> 2);
      L.brd_kn[nb] = (uint32_t)(kr * P::kBKRowBytes + (((n >> 3) ^ swz_krow(kr)) << 4) + ((n >> 2) & 1) * 8);
    }
  }

  L.srd = (uint32_t)(wave * kTileN + wave_n * 64 + (lane & 31));

  f32x16_t acc[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

  // the tile's 32-row blocks are split evenly between the two wave rows
  // (a 192-row chunk runs 3 + 3 blocks, not 4 + 2); a wave's rows start at
  // row0 of the tile
  const int mblk = ceil_div(min(t.mcount, kChunkRows), 32);
  const int msplit = (mblk + 1) >> 1;
  const int row0 = wave_m * msplit * 32;
  const int mbn = wave_m == 0 ? msplit : mblk - msplit;
  const int ncols = t.N - (t.n0 + wave_n * 64);
  const int nbn = mbn == 0 ? 0 : (ncols >= 64 ? 2 : (ncols > 0 ? ceil_div(ncols, 32) : 0));
  const char* Ab = (const char*)A;
#define MOE_LOOP(MB_, NB_) mfma_loop<BMODE, MB_, NB_, WF, SPLIT>(t, L, Ab, Bb, Sb, smem, wave, row0, lane, acc)
  switch (nbn * 4 + (max(mbn, 1) - 1)) {
    case 0: case 1: case 2: case 3: MOE_LOOP(4, 0); break;
    case 4: MOE_LOOP(1, 1); break;
    case 5: MOE_LOOP(2, 1); break;
    case 6: MOE_LOOP(3, 1); break;
    case 7: MOE_LOOP(4, 1); break;
    case 8: MOE_LOOP(1, 2); break;
    case 9: MOE_LOOP(2, 2); break;
    case 10: MOE_LOOP(3, 2); break;
    default: MOE_LOOP(4, 2); break;
  }
#undef MOE_LOOP
  // FP8 B: the output column's scale, applied to the fp32 sum first
  float bsc[2] = {1.0f, 1.0f};
  if (W8)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int col = t.n0 + wave_n * 64 + nb * 32 + (lane & 31);
      bsc[nb] = col < t.N ? t.bscale[col] : 0.0f;
    }
  bool mact[4], nact[2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) mact[mb] = mb < mbn;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) nact[nb] = nb < nbn;
  const bool wave_active = nbn > 0;

  // ---- epilogue ----
  // accumulator layout of the 32x32 MFMA: lane l, register r holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32, of the wave's rows from row0
  if (t.cf32) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if (!mact[mb]) continue;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        if (!nact[nb]) continue;
        const int col = t.n0 + wave_n * 64 + nb * 32 + (lane & 31);
        if (col >= t.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < t.mcount)
            epilogue_store<EPI, BMODE == B_NKP || BMODE == B_KN>(a, t, row, col, W8 ? acc[mb][nb][r] * bsc[nb] : acc[mb][nb][r]);
        }
      }
    }
    return;
  }
  // bf16: stage the wave's 128 x 64 block in LDS, then store 16-byte rows
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (!wave_active) return;
  uint16_t* stage = (uint16_t*)(smem + wave * (128 * 64 * 2));
  if (EPI == EPI_DRELU2) {
    // the forward's h of the block, read in 16-byte rows into the staging
    // area (the layout the stores below read); each lane then takes its
    // elements' h from there and overwrites them with its results
    const uint16_t* Hf = (const uint16_t*)t.aux;
#pragma unroll 4
    for (int it = 0; it < 128 * 8 / 64; ++it) {
      const int id = it * 64 + lane;
      const int lr = id >> 3, c = id & 7;
      const int col = t.n0 + wave_n * 64 + c * 8;
      if (lr < mbn * 32 && row0 + lr < t.mcount && col < t.N)
        *(uint4*)(stage + lr * 64 + c * 8) = *(const uint4*)(Hf + (t.rowbase + t.m0 + row0 + lr) * t.ldc + col);
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  }
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if (!mact[mb]) continue;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int lc = nb * 32 + (lane & 31);
      const int col = t.n0 + wave_n * 64 + lc;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        float v = W8 ? acc[mb][nb][r] * bsc[nb] : acc[mb][nb][r];
        if (EPI == EPI_DRELU2)
          v *= 2.0f * sqrtf(bf16_to_f32(stage[lr * 64 + lc]));  // rows and columns past the tile are not stored
        else if (EPI != EPI_STORE && row0 + lr < t.mcount && col < t.N)
          v = epilogue_value<EPI>(a, t, t.rowbase + t.m0 + row0 + lr, col, v);
        stage[lr * 64 + lc] = (uint16_t)f32_to_bf16(v);
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

// ---------------------------------------------------------------------------
// Split-K bf16 kernel for dense launches with K periods (the router's bf16x3
// GEMM): 128 x 128 tiles, register-staged double-buffered LDS.
// ---------------------------------------------------------------------------
constexpr int kLdsStride = 72;  // 64 K-values + 8 pad (bf16): 144-byte rows, conflict-free b128 reads

__global__ __launch_bounds__(256, 2) void gemm_bf16_splitk_kernel(GemmArgs a) {
  __shared__ __align__(16) uint16_t sA[2][kDenseChunkRows * kLdsStride];
  __shared__ __align__(16) uint16_t sB[2][kDenseTileN * kLdsStride];

  Tile t;
  if (!decode_tile(a, t, kDenseChunkRows, kDenseTileN)) return;
  const uint16_t* A = (const uint16_t*)t.A;
  const uint16_t* B = (const uint16_t*)t.B;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int a_period = a.a_period;

  const int ck = tid & 7, r0 = tid >> 3;
  const uint16_t* arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) arow[i] = A + src_row(t, r0 + 32 * i) * t.lda + ck * 8;
  const uint16_t* brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int n = t.n0 + r0 + 32 * i;
    n = n < t.N ? n : t.N - 1;
    brow[i] = B + (long)n * t.ldb + ck * 8;
  }

  uint4 ra[4], rb[4];
  auto load = [&](int kt) {
    const int k0 = kt * 64;
    const bool kin = k0 + ck * 8 < t.Kd;
    const int ka = a_period ? (k0 % a_period) : k0;
    const bool ain = a_period ? (ka + ck * 8 < a.a_cols) : kin;
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = ain ? *(const uint4*)(arow[i] + ka) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[i] = kin ? *(const uint4*)(brow[i] + k0) : make_uint4(0, 0, 0, 0);
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *(uint4*)&sA[buf][(r0 + 32 * i) * kLdsStride + ck * 8] = ra[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) *(uint4*)&sB[buf][(r0 + 32 * i) * kLdsStride + ck * 8] = rb[i];
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

  bool mact[2], nact[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) mact[mb] = wm * 64 + mb * 32 < t.mcount;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) nact[nb] = t.n0 + wn * 64 + nb * 32 < t.N;

  if (t.k_begin < t.k_end) {
    load(t.k_begin);
    store(0);
    __syncthreads();
    for (int kt = t.k_begin; kt < t.k_end; ++kt) {
      const int buf = (kt - t.k_begin) & 1;
      const bool more = kt + 1 < t.k_end;
      if (more) load(kt + 1);
      // every block is computed: rows past the chunk and columns past N
      // hold clamped copies in LDS, and the epilogue stores only the valid
      // blocks (a branch per MFMA would serialise the loop)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int koff = kk * 16 + (lane >> 5) * 8;
        uint4 af[2], bf[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          af[mb] = *(const uint4*)&sA[buf][(wm * 64 + mb * 32 + (lane & 31)) * kLdsStride + koff];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          bf[nb] = *(const uint4*)&sB[buf][(wn * 64 + nb * 32 + (lane & 31)) * kLdsStride + koff];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma_32x32x16(af[mb], bf[nb], acc[mb][nb]);
      }
      if (more) store(buf ^ 1);
      __syncthreads();
    }
  }

#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    if (!mact[mb]) continue;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      if (!nact[nb]) continue;
      const int col = t.n0 + wn * 64 + nb * 32 + (lane & 31);
      if (col >= t.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < t.mcount) epilogue_store<EPI_STORE>(a, t, row, col, acc[mb][nb][r]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel (plain FMAs): 128-row x kTileN-column tiles, computed as
// 128 x 128 halves
// ---------------------------------------------------------------------------
template <int BMODE, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  __shared__ float sA[16][128 + 4];
  __shared__ float sB[16][128 + 4];
  Tile t;
  if (!decode_tile(a, t, kChunkRows, kTileN)) return;
  const float* A = (const float*)t.A;
  const float* B = (const float*)t.B;
  if (t.g > 0) B += (long)(t.g - 1) * a.strideB;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int a_period = (t.g == 0) ? a.a_period : 0;
  const int lr = tid >> 1, kh = (tid & 1) * 8;

  // the tile as 128 x 128 blocks
  for (int mh = 0; mh < kChunkRows / 128; ++mh) {
    const int mrow0 = mh * 128;
    if (mrow0 >= t.mcount) break;
    const float* arow = A + src_row(t, mrow0 + lr) * t.lda + kh;
    for (int half = 0; half < kTileN / 128; ++half) {
      const int n0 = t.n0 + half * 128;
      if (n0 >= t.N) break;
      float acc[8][8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

      const int kbeg = t.k_begin * 64, kend = min(t.Kd, t.k_end * 64);
      for (int k0 = kbeg; k0 < kend; k0 += 16) {
        const int ka = a_period ? (k0 % a_period) : k0;
#pragma unroll
        for (int q = 0; q < 8; ++q) sA[kh + q][lr] = (k0 + kh + q < t.Kd) ? arow[ka + q] : 0.0f;
        if (BMODE == B_NK) {
          int n = n0 + lr;
          n = n < t.N ? n : t.N - 1;
          const float* brow = B + (long)n * t.ldb + kh;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int k = k0 + kh + q;
            sB[kh + q][lr] = k >= t.Kd ? 0.0f
                             : a.b_packed ? B[packed_out_in_offset(n, k, t.N, t.Kd)]
                                          : brow[k0 + q];
          }
        } else {
          const int kr = tid >> 4, nc = (tid & 15) * 8;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int n = n0 + nc + q;
            float v = 0.0f;
            if (k0 + kr < t.Kd && n < t.N)
              v = a.b_packed ? B[packed_neuron_major_offset(k0 + kr, n, t.Kd, t.N)]
                             : B[(long)(k0 + kr) * t.ldb + n];
            sB[kr][nc + q] = v;
          }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          float av[8], bv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) av[i] = sA[k][ty + 16 * i];
#pragma unroll
          for (int j = 0; j < 8; ++j) bv[j] = sB[k][tx + 16 * j];
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
        }
        __syncthreads();
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = mrow0 + ty + 16 * i;
        if (row >= t.mcount) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int col = n0 + tx + 16 * j;
          if (col < t.N) epilogue_store<EPI>(a, t, row, col, acc[i][j]);
        }
      }
    }
  }
}

hipError_t launch_gemm(const GemmArgs& a, int act_bf16, int b_mode, int epi, int max_tiles,
                       hipStream_t s) {
  const bool splitk = act_bf16 && !a.split_main && (a.ksplit > 1 || a.a_period);
  if (splitk) {
    if (a.plan || b_mode != B_NK || epi != EPI_STORE) return hipErrorInvalidValue;
    const int tiles = ceil_div(a.M_s, kDenseChunkRows) * ceil_div(a.N_s, kDenseTileN) * (a.ksplit > 1 ? a.ksplit : 1);
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_bf16_splitk_kernel, dim3(xcd_grid(tiles)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (act_bf16 && ((a.ksplit > 1 && (a.plan || !a.split_main || !a.c_s_f32 || epi != EPI_STORE)) ||
                   (!a.b_packed && b_mode != B_NKP)))
    return hipErrorInvalidValue;
  if ((a.b_fp8 || a.b_fp4) && (!act_bf16 || a.plan == nullptr)) return hipErrorInvalidValue;
  if (a.b_fp4 && (a.b_fp8 || b_mode != B_NK || !a.e8 || a.Kd % kMxBlock || a.N % kMxBlock ||
                  (a.M_s > 0 && (!a.e8_s || a.Kd_s % kMxBlock || a.N_s % kMxBlock))))
    return hipErrorInvalidValue;
  if ((b_mode == B_NKP) != (a.wgrad != 0) || (a.wgrad && (!act_bf16 || epi != EPI_STORE)))
    return hipErrorInvalidValue;
  int grid;
  if (a.wgrad) {
    const int tpr = ceil_div(a.M, kChunkRows) * ceil_div(a.N, kTileN);
    const int tps = a.Kd_s > 0 ? ceil_div(a.M_s, kChunkRows) * ceil_div(a.N_s, kTileN) : 0;
    if (a.E * tpr + tps == 0) return hipSuccess;
    grid = wgrad_grid(a.E, tpr, tps);
  } else if (a.plan) {
    grid = xcd_grid(max_tiles);
  } else {
    const int tiles = ceil_div(a.M_s, kChunkRows) * ceil_div(a.N_s, kTileN) * (a.ksplit > 1 ? a.ksplit : 1);
    if (tiles == 0) return hipSuccess;
    grid = xcd_grid(tiles);
  }
  dim3 g(grid), b(256), bm(kThreads);
  if (a.b_fp8) {
    if (b_mode == B_NK && epi == EPI_RELU2)
      hipLaunchKernelGGL((gemm_bf16_mfma_kernel<B_NK, EPI_RELU2, 1>), g, bm, 0, s, a);
    else if (b_mode == B_KN && epi == EPI_STORE)
      hipLaunchKernelGGL((gemm_bf16_mfma_kernel<B_KN, EPI_STORE, 1>), g, bm, 0, s, a);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (a.b_fp4) {
    if (epi == EPI_RELU2)
      hipLaunchKernelGGL((gemm_bf16_mfma_kernel<B_NK, EPI_RELU2, 2>), g, bm, 0, s, a);
    else if (epi == EPI_STORE)
      hipLaunchKernelGGL((gemm_bf16_mfma_kernel<B_NK, EPI_STORE, 2>), g, bm, 0, s, a);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (a.split_main && a.ksplit > 1) {
    // a dense launch split over K: fp32 partials (checked above)
    if (!act_bf16 || b_mode != B_NK) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_bf16_mfma_kernel<B_NK, EPI_STORE, 0, true>), g, bm, 0, s, a);
    return hipGetLastError();
  }
#define MOE_GEMM_CASE(BM, EP)                                                        \
  if (b_mode == BM && epi == EP) {                                                   \
    if (act_bf16)                                                                    \
      hipLaunchKernelGGL((gemm_bf16_mfma_kernel<BM, EP, 0>), g, bm, 0, s, a);    \
    else                                                                             \
      hipLaunchKernelGGL((gemm_f32_kernel<BM, EP>), g, b, 0, s, a);                  \
    return hipGetLastError();                                                        \
  }
  MOE_GEMM_CASE(B_NK, EPI_RELU2)
  MOE_GEMM_CASE(B_NK, EPI_STORE)
  MOE_GEMM_CASE(B_NK, EPI_ADD_F32)
  MOE_GEMM_CASE(B_KN, EPI_STORE)
  if (act_bf16 && b_mode == B_KN && epi == EPI_DRELU2) {
    hipLaunchKernelGGL((gemm_bf16_mfma_kernel<B_KN, EPI_DRELU2, 0>), g, bm, 0, s, a);
    return hipGetLastError();
  }
  if (b_mode == B_NKP && epi == EPI_STORE) {
    hipLaunchKernelGGL((gemm_bf16_mfma_kernel<B_NKP, EPI_STORE, 0>), g, bm, 0, s, a);
    return hipGetLastError();
  }
#undef MOE_GEMM_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
