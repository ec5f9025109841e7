// Grouped GEMMs of the routed experts, the shared expert and the dense
// projections (router in bf16x3 form, latent in/out).
//
// bf16 path: MFMA v_mfma_f32_32x32x16_bf16 on CDNA4.  A workgroup of 4
// waves computes a 128-row x 128-column tile; each wave owns a 64 x 64
// quarter as 2 x 2 MFMA blocks of 32 x 32 with fp32 accumulators.  K runs in
// steps of 64: the A rows (gathered through the route map for routed
// experts, so the packed [R, d] input is never materialised) and the weight
// tile are staged in LDS, double-buffered, with the next step's global loads
// in flight while the MFMAs of the current step run.  Weights stored [K][N]
// (the neuron-major down projections) are transposed in registers 8 x 4 at a
// time on their way into LDS, so both operands are read as 16-byte
// K-contiguous fragments.
//
// fp32 path (the tiny fp32 layer): the same tiles computed with plain fp32
// FMAs, 8 x 8 outputs per thread.
//
// Epilogues: ReLU^2 with the rounding points bf16(relu(bf16(u))^2) of the
// NemotronH "Arithmetic" section (plain relu(u)^2 in fp32); plain store
// (bf16 or fp32); add an fp32 addend (and optionally the old output) before
// the single rounding.
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kLdsStride = 72;  // 64 K-values + 8 pad (bf16): 144-byte rows, conflict-free b128 reads

__device__ __forceinline__ f32x16_t mfma_32x32x16(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

struct Tile {
  int g, m0, mcount, n0, N, Kd, k_begin, k_end;
  long rowbase;
  const void* A;
  long lda;
  const void* B;
  long ldb;
  void* C;
  long ldc;
  int cf32;
  const int32_t* gather;
  int gdiv;
};

// Decode the workgroup's tile; returns false when it has none.
__device__ __forceinline__ bool decode_tile(const GemmArgs& a, Tile& t) {
  const int tile = xcd_tile_of(blockIdx.x);
  int ch, nt, ks = 0;
  if (a.plan) {
    if (tile >= *a.num_tiles) return false;
    t.g = a.plan[2 * tile];
    const int v = a.plan[2 * tile + 1];
    ch = v >> 16;
    nt = v & 0xffff;
  } else {
    const int nch = ceil_div(a.M_s, kChunkRows), ntc = ceil_div(a.N_s, kTileN);
    const int per = nch * ntc;
    if (tile >= per * max(1, a.ksplit)) return false;
    t.g = 0;
    ks = tile / per;
    plan_decode_local(tile - ks * per, nch, ntc, &ch, &nt);
  }
  int count;
  if (t.g == 0) {
    t.rowbase = 0;
    count = a.M_s;
    t.A = a.A_s;
    t.lda = a.lda_s;
    t.B = a.B_s;
    t.ldb = a.ldb_s;
    t.N = a.N_s;
    t.Kd = a.Kd_s;
    t.C = a.C_s;
    t.ldc = a.ldc_s;
    t.cf32 = a.c_s_f32;
    t.gather = nullptr;
    t.gdiv = 1;
  } else {
    const int e = t.g - 1;
    t.rowbase = a.offsets[e];
    count = a.offsets[e + 1] - (int)t.rowbase;
    t.A = a.A;
    t.lda = a.lda;
    t.B = a.B;  // expert offset applied by the element-typed caller
    t.ldb = a.ldb;
    t.N = a.N;
    t.Kd = a.Kd;
    t.C = a.C;
    t.ldc = a.ldc;
    t.cf32 = a.c_f32;
    t.gather = a.gather;
    t.gdiv = a.gdiv;
  }
  t.m0 = ch * kChunkRows;
  t.mcount = min(kChunkRows, count - t.m0);
  t.n0 = nt * kTileN;
  if (t.mcount <= 0) return false;
  // K range in steps of 64 (split-K for dense launches)
  const int nk = ceil_div(t.Kd, 64);
  if (a.plan || a.ksplit <= 1) {
    t.k_begin = 0;
    t.k_end = nk;
  } else {
    const int per = ceil_div(nk, a.ksplit);
    t.k_begin = min(nk, ks * per);
    t.k_end = min(nk, t.k_begin + per);
    t.C = (char*)t.C + (long)ks * a.split_stride * (t.cf32 ? 4 : 2);
  }
  return true;
}

// Source row of local row m (clamped into the chunk so every load is valid).
__device__ __forceinline__ long src_row(const Tile& t, int m) {
  const int mm = m < t.mcount ? m : t.mcount - 1;
  const long j = t.rowbase + t.m0 + mm;
  return t.gather ? (long)(t.gather[j] / t.gdiv) : j;
}

template <int EPI>
__device__ __forceinline__ void epilogue_store(const GemmArgs& a, const Tile& t, int row, int col,
                                               float v) {
  const long orow = t.rowbase + t.m0 + row;
  if (EPI == EPI_RELU2) {
    if (t.cf32) {
      const float r = fmaxf(v, 0.0f);
      ((float*)t.C)[orow * t.ldc + col] = r * r;
    } else {
      const float r = fmaxf(bf16_round(v), 0.0f);
      ((uint16_t*)t.C)[orow * t.ldc + col] = (uint16_t)f32_to_bf16(r * r);
    }
  } else {
    if (EPI == EPI_ADD_F32) {
      if (a.addend) v += a.addend[orow * a.ld_add + col];
      if (a.accumulate)
        v += t.cf32 ? ((const float*)t.C)[orow * t.ldc + col]
                    : bf16_to_f32(((const uint16_t*)t.C)[orow * t.ldc + col]);
    }
    if (t.cf32)
      ((float*)t.C)[orow * t.ldc + col] = v;
    else
      ((uint16_t*)t.C)[orow * t.ldc + col] = (uint16_t)f32_to_bf16(v);
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
template <int BMODE, int EPI>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmArgs a) {
  __shared__ __align__(16) uint16_t sA[2][kChunkRows * kLdsStride];
  __shared__ __align__(16) uint16_t sB[2][kTileN * kLdsStride];

  Tile t;
  if (!decode_tile(a, t)) return;
  const uint16_t* A = (const uint16_t*)t.A;
  const uint16_t* B = (const uint16_t*)t.B;
  if (t.g > 0) B += (long)(t.g - 1) * a.strideB;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int a_period = (t.g == 0) ? a.a_period : 0;

  // A rows: thread loads 16-byte chunk ck of rows r0 + 32 i
  const int ck = tid & 7, r0 = tid >> 3;
  const uint16_t* arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) arow[i] = A + src_row(t, r0 + 32 * i) * t.lda + ck * 8;

  // B: NK -> rows n0 + r0 + 32 i; KN -> an 8 (k) x 4 (n) block per thread
  const uint16_t* brow[4];
  const uint16_t* bkn = nullptr;
  bool bkn_ok = false;
  const int fo = tid >> 5, cq = tid & 31;
  if (BMODE == B_NK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int n = t.n0 + r0 + 32 * i;
      n = n < t.N ? n : t.N - 1;
      brow[i] = B + (long)n * t.ldb + ck * 8;
    }
  } else {
    const int col = t.n0 + 4 * cq;
    bkn_ok = col < t.N;
    bkn = B + (long)(8 * fo) * t.ldb + (bkn_ok ? col : 0);
  }

  uint4 ra[4];
  uint4 rbn[4];
  uint2 rbk[8];
  auto load = [&](int kt) {
    const int k0 = kt * 64;
    const bool kin = k0 + ck * 8 < t.Kd;
    const int ka = a_period ? (k0 % a_period) : k0;
    const bool ain = a_period ? (ka + ck * 8 < a.a_cols) : kin;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[i] = ain ? *(const uint4*)(arow[i] + ka) : make_uint4(0, 0, 0, 0);
    if (BMODE == B_NK) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        rbn[i] = kin ? *(const uint4*)(brow[i] + k0) : make_uint4(0, 0, 0, 0);
    } else {
      const bool ok = bkn_ok && (k0 + 8 * fo < t.Kd);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        rbk[i] = ok ? *(const uint2*)(bkn + (long)(k0 + i) * t.ldb) : make_uint2(0, 0);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(uint4*)&sA[buf][(r0 + 32 * i) * kLdsStride + ck * 8] = ra[i];
    if (BMODE == B_NK) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(uint4*)&sB[buf][(r0 + 32 * i) * kLdsStride + ck * 8] = rbn[i];
    } else {
      // rbk[i] = row k0+8fo+i, columns 4cq..4cq+3 -> column j holds 8 k-values
      uint4 c0, c1, c2, c3;
      c0.x = (rbk[0].x & 0xffffu) | (rbk[1].x << 16);
      c0.y = (rbk[2].x & 0xffffu) | (rbk[3].x << 16);
      c0.z = (rbk[4].x & 0xffffu) | (rbk[5].x << 16);
      c0.w = (rbk[6].x & 0xffffu) | (rbk[7].x << 16);
      c1.x = (rbk[0].x >> 16) | (rbk[1].x & 0xffff0000u);
      c1.y = (rbk[2].x >> 16) | (rbk[3].x & 0xffff0000u);
      c1.z = (rbk[4].x >> 16) | (rbk[5].x & 0xffff0000u);
      c1.w = (rbk[6].x >> 16) | (rbk[7].x & 0xffff0000u);
      c2.x = (rbk[0].y & 0xffffu) | (rbk[1].y << 16);
      c2.y = (rbk[2].y & 0xffffu) | (rbk[3].y << 16);
      c2.z = (rbk[4].y & 0xffffu) | (rbk[5].y << 16);
      c2.w = (rbk[6].y & 0xffffu) | (rbk[7].y << 16);
      c3.x = (rbk[0].y >> 16) | (rbk[1].y & 0xffff0000u);
      c3.y = (rbk[2].y >> 16) | (rbk[3].y & 0xffff0000u);
      c3.z = (rbk[4].y >> 16) | (rbk[5].y & 0xffff0000u);
      c3.w = (rbk[6].y >> 16) | (rbk[7].y & 0xffff0000u);
      uint16_t* dst = &sB[buf][(4 * cq) * kLdsStride + 8 * fo];
      *(uint4*)(dst + 0 * kLdsStride) = c0;
      *(uint4*)(dst + 1 * kLdsStride) = c1;
      *(uint4*)(dst + 2 * kLdsStride) = c2;
      *(uint4*)(dst + 3 * kLdsStride) = c3;
    }
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
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int koff = kk * 16 + (lane >> 5) * 8;
        uint4 af[2], bf[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          if (mact[mb])
            af[mb] = *(const uint4*)&sA[buf][(wm * 64 + mb * 32 + (lane & 31)) * kLdsStride + koff];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          if (nact[nb])
            bf[nb] = *(const uint4*)&sB[buf][(wn * 64 + nb * 32 + (lane & 31)) * kLdsStride + koff];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            if (mact[mb] && nact[nb]) acc[mb][nb] = mfma_32x32x16(af[mb], bf[nb], acc[mb][nb]);
      }
      if (more) store(buf ^ 1);
      __syncthreads();
    }
  }

  // accumulator layout of the 32x32 MFMA: lane l, register r holds
  // row 8*(r/4) + 4*(l/32) + r%4, column l%32
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
        if (row < t.mcount) epilogue_store<EPI>(a, t, row, col, acc[mb][nb][r]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel (plain FMAs), same tiles
// ---------------------------------------------------------------------------
template <int BMODE, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  __shared__ float sA[16][kChunkRows + 4];
  __shared__ float sB[16][kTileN + 4];
  Tile t;
  if (!decode_tile(a, t)) return;
  const float* A = (const float*)t.A;
  const float* B = (const float*)t.B;
  if (t.g > 0) B += (long)(t.g - 1) * a.strideB;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int a_period = (t.g == 0) ? a.a_period : 0;

  // A: thread loads row lr = tid / 2, k-half (tid & 1) * 8
  const int lr = tid >> 1, kh = (tid & 1) * 8;
  const float* arow = A + src_row(t, lr) * t.lda + kh;
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
      int n = t.n0 + lr;
      n = n < t.N ? n : t.N - 1;
      const float* brow = B + (long)n * t.ldb + kh;
#pragma unroll
      for (int q = 0; q < 8; ++q) sB[kh + q][lr] = (k0 + kh + q < t.Kd) ? brow[k0 + q] : 0.0f;
    } else {
      const int kr = tid >> 4, nc = (tid & 15) * 8;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int n = t.n0 + nc + q;
        sB[kr][nc + q] = (k0 + kr < t.Kd && n < t.N) ? B[(long)(k0 + kr) * t.ldb + n] : 0.0f;
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
    const int row = ty + 16 * i;
    if (row >= t.mcount) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = t.n0 + tx + 16 * j;
      if (col < t.N) epilogue_store<EPI>(a, t, row, col, acc[i][j]);
    }
  }
}

hipError_t launch_gemm(const GemmArgs& a, int act_bf16, int b_mode, int epi, int max_tiles,
                       hipStream_t s) {
  int grid;
  if (a.plan) {
    grid = xcd_grid(max_tiles);
  } else {
    const int tiles = ceil_div(a.M_s, kChunkRows) * ceil_div(a.N_s, kTileN) * (a.ksplit > 1 ? a.ksplit : 1);
    if (tiles == 0) return hipSuccess;
    grid = xcd_grid(tiles);
  }
  dim3 g(grid), b(256);
#define MOE_GEMM_CASE(BM, EP)                                                        \
  if (b_mode == BM && epi == EP) {                                                   \
    if (act_bf16)                                                                    \
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, EP>), g, b, 0, s, a);                 \
    else                                                                             \
      hipLaunchKernelGGL((gemm_f32_kernel<BM, EP>), g, b, 0, s, a);                  \
    return hipGetLastError();                                                        \
  }
  MOE_GEMM_CASE(B_NK, EPI_RELU2)
  MOE_GEMM_CASE(B_NK, EPI_STORE)
  MOE_GEMM_CASE(B_NK, EPI_ADD_F32)
  MOE_GEMM_CASE(B_KN, EPI_STORE)
#undef MOE_GEMM_CASE
  return hipErrorInvalidValue;
}

}  // namespace moe
