// The tile a workgroup of the grouped GEMMs computes: which group (the shared
// expert or a routed expert), which row chunk and column tile, and the
// operand pointers of that group.  Shared by the bf16 / FP8 / MXFP4-weight
// kernel (gemm.hip) and the MXFP8-activation kernel (mxgemm.hip).
#pragma once

#include "moe_internal.h"

namespace moe {

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
  const float* bscale;  // FP8 B: scale of output column n at bscale[n]
  const uint8_t* e8;    // MXFP4 B: E8M0 scales [Kd / 32][N], block j of column n at e8[j * N + n]
  const void* aux;      // EPI_DRELU2: the forward's h, C's layout
  const uint8_t* as;    // MXFP8 A: scales of the group, block j of row r at as[j * ld_as + r]
  long ld_as;
  uint8_t* cs;          // EPI_QRELU2: output scales, block j of row r at cs[j * ld_cs + r]
  long ld_cs;
};

// Decode the workgroup's tile (row chunks of tile_m, column tiles of tile_n);
// returns false when it has none.
__device__ __forceinline__ bool decode_tile(const GemmArgs& a, Tile& t, int tile_m, int tile_n) {
  int tile = xcd_tile_of(blockIdx.x);
  int ch, nt, ks = 0;
  if (a.wgrad) {
    // weight gradients: tiles [0, tps) of group 0, then E groups of tpr
    // tiles (expert e: tps + e tpr + l)
    const int tpr = ceil_div(a.M, tile_m) * ceil_div(a.N, tile_n);
    const int tps = a.Kd_s > 0 ? ceil_div(a.M_s, tile_m) * ceil_div(a.N_s, tile_n) : 0;
    tile = wgrad_tile_of(blockIdx.x, a.E, tpr, tps);
    if (tile < 0) return false;
    int l, count;
    if (tile < tps) {
      t.g = 0;
      l = tile;
      nt = ceil_div(a.N_s, tile_n);
      t.A = a.A_s;
      t.lda = a.lda_s;
      t.B = a.B_s;
      t.ldb = a.ldb_s;
      t.N = a.N_s;
      t.Kd = a.Kd_s;
      t.C = a.C_s;
      t.ldc = a.ldc_s;
      count = a.M_s;
    } else {
      const int e = (tile - tps) / tpr;
      l = tile - tps - e * tpr;
      nt = ceil_div(a.N, tile_n);
      const int k0 = a.koff[e];
      t.g = e + 1;
      t.A = (const uint16_t*)a.A + k0;
      t.lda = a.lda;
      t.B = (const uint16_t*)a.B + k0;
      t.ldb = a.ldb;
      t.N = a.N;
      t.Kd = a.koff[e + 1] - k0;
      t.C = (float*)a.C + (long)e * a.M * a.N;
      t.ldc = a.N;
      count = a.M;
    }
    ch = l / nt;
    nt = l - ch * nt;
    t.rowbase = 0;
    t.m0 = ch * tile_m;
    t.mcount = min(tile_m, count - t.m0);
    t.n0 = nt * tile_n;
    t.cf32 = 1;
    t.gather = nullptr;
    t.gdiv = 1;
    t.bscale = nullptr;
    t.e8 = nullptr;
    t.aux = nullptr;
    t.as = nullptr;
    t.ld_as = 0;
    t.cs = nullptr;
    t.ld_cs = 0;
    t.k_begin = 0;
    t.k_end = ceil_div(t.Kd, 64);
    return t.mcount > 0;
  }
  if (a.plan) {
    if (tile >= *a.num_tiles) return false;
    t.g = a.plan[2 * tile];
    const int v = a.plan[2 * tile + 1];
    ch = v >> 16;
    nt = v & 0xffff;
  } else {
    const int nch = ceil_div(a.M_s, tile_m), ntc = ceil_div(a.N_s, tile_n);
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
    t.bscale = a.bscale_s;
    t.e8 = a.e8_s;
    t.aux = a.aux_s;
    t.as = a.as_s;
    t.ld_as = a.ld_as_s;
    t.cs = a.cs_s;
    t.ld_cs = a.ld_cs_s;
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
    t.bscale = a.bscale ? a.bscale + (long)e * a.N : nullptr;
    t.e8 = a.e8 ? a.e8 + (long)e * a.N * (a.Kd / kMxBlock) : nullptr;
    t.aux = a.aux;
    t.as = a.as;
    t.ld_as = a.ld_as;
    t.cs = a.cs;
    t.ld_cs = a.ld_cs;
  }
  t.m0 = ch * tile_m;
  t.mcount = min(tile_m, count - t.m0);
  t.n0 = nt * tile_n;
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

// s_waitcnt vmcnt(N)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ int swz_rows(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int swz_krow(int k) { return (0xEA40 >> ((k & 3) * 4)) & 15; }

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Direct global->LDS load of 16 bytes per lane: lane i's bytes land at LDS
// address lds + 16 i (lds wave-uniform).  Written as inline assembly so the
// compiler does not see an LDS write it would have to wait for before every
// LDS read; the K loop tracks these loads with explicit vmcnt waits instead.
// The kernel itself makes no other use of M0.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds), "v"(voff), "s"(base) : "memory");
}

// Direct global->LDS load of 4 bytes per lane (lane i at lds + 4 i).
__device__ __forceinline__ void lds_dma4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(lds), "v"(voff), "s"(base) : "memory");
}

}  // namespace moe
