// The C ABI of libmoe (declared in include/moe.h): host-side argument
// checks, workspace carving and the launch sequence of each call.  No call
// allocates device memory, synchronises the host or keeps state.
#include <limits.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "moe_internal.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
constexpr long kMaxRoutes = 1L << 22;  // chunk index of the tile plan fits 15 bits
constexpr int kMaxWidth = 8192;        // combine: one thread per 8 columns, <= 1024 threads

struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <class T>
  T* take(size_t n) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    T* p = base ? (T*)(base + off) : nullptr;
    off += n * sizeof(T);
    return p;
  }
};

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t act_size(moe_dtype dt) { return dt == MOE_BF16 ? 2 : 4; }
inline moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY2(expr)                     \
  do {                                     \
    const moe_status _st = (expr);         \
    if (_st != MOE_OK) return _st;         \
  } while (0)

#define MOE_TRY(expr)                          \
  do {                                         \
    const hipError_t _e = (expr);              \
    if (_e != hipSuccess) return MOE_ERR_HIP;  \
  } while (0)

// Router constraints ("Nemotron is not one circuit", "The Router Is A
// Deterministic Algorithm": equal groups, top-2 group score, top-K of the
// surviving experts).
moe_status check_router(int T, int E, int K, int n_group, int topk_group) {
  if (T < 0 || E < 1 || K < 1 || K > E) return MOE_ERR_INVALID_ARG;
  if (n_group < 1 || E % n_group != 0) return MOE_ERR_INVALID_ARG;
  if (topk_group < 1 || topk_group > n_group) return MOE_ERR_INVALID_ARG;
  if (n_group > 1 && E / n_group < 2) return MOE_ERR_INVALID_ARG;
  if ((long)K > (long)topk_group * (E / n_group)) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || K > MOE_MAX_TOPK || n_group > MOE_MAX_GROUPS) return MOE_ERR_UNSUPPORTED;
  if ((long)T * K > kMaxRoutes) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The grouped GEMMs address each activation operand (x, the latent x, h,
// h_s, y_lat) through 32-bit byte offsets from the matrix base, and the
// combine reads y_packed and y_s likewise; a matrix of 2^32 bytes or more
// would wrap silently, so such sizes are rejected (MOE_ERR_UNSUPPORTED).
constexpr long kMaxOperandBytes = 1L << 32;
// A weight matrix is packed and addressed per expert with 32-bit offsets;
// moe_pack_weight accepts at most 2^31 bytes per matrix.
constexpr long kMaxWeightBytes = 1L << 31;
// The decode path's work items carry a 12-bit chunk index.
constexpr int kMaxDecodeChunks = 1 << 12;

inline bool fits_operand(long rows, long width, long eb) { return rows * width * eb < kMaxOperandBytes; }

// Whether a fused forward call runs the decode path (live-neuron skipping):
// requested by MOE_FLAG_ZERO_SKIP_DOWN, for bf16 batches of at most
// kDecodeMaxRows rows and kDecodeMaxRoutes routes.  Otherwise the flag is a
// hint only and the grouped GEMMs run; the result is the same layer.
bool decode_path(const moe_layer_desc* d, int T) {
  return (d->flags & MOE_FLAG_ZERO_SKIP_DOWN) && d->act_dtype == MOE_BF16 && T <= kDecodeMaxRows &&
         (long)T * d->K <= kDecodeMaxRoutes && d->d <= kDecodeMaxWidth && d->d_latent <= kDecodeMaxWidth &&
         ceil_div(d->F, kDecodeChunk) <= kMaxDecodeChunks && ceil_div(d->F_shared, kDecodeChunk) <= kMaxDecodeChunks &&
         !(d->flags & MOE_FLAG_MXFP8_ACTIVATIONS) && !(d->capacity_factor > 0.0f);
}

// K splits of a dense bf16 latent projection ([T, N] output, K = Kd) on the
// 256 x 256 GEMM: doubled while the launch stays within 256 workgroups and
// each split keeps at least 256 of K (fp32 partials, then one reduction).
int latent_splits(int T, int N, int Kd) {
  const int tiles = ceil_div(T, kChunkRows) * ceil_div(N, kTileN);
  int S = 1;
  while (tiles * S * 2 <= 256 && Kd / (64 * S * 2) >= 4) S *= 2;
  return S;
}

// Route slots per expert for a capacity factor: ceil(CF * T * K / E) in
// double ("M6.1 - Routed Capacity", 0x06), or -1 when it does not fit an int.
long capacity_slots(int T, int K, int E, float cf) {
  const double c = ceil((double)cf * T * K / E);
  return c > (double)INT_MAX ? -1 : (long)c;
}

// Buffers of moe_layer_forward, carved from the workspace in a fixed order.
struct FwdBufs {
  bool decode;
  float* logits;
  uint16_t* w3;
  int S;
  int32_t *ids, *counts, *offsets, *route_src, *route_pos;
  float* wts;
  void* dscratch;
  int32_t *plan_up, *plan_down, *num_tiles;
  long max_up, max_down;
  void *x_norm, *x_lat, *h, *h_s, *y_packed, *y_lat;
  float* y_s;
  // bf16 latent projections split over K: their fp32 partials
  int S_lin, S_lout;
  float* part_lat;
  // the capacity-bounded variant: the dropless dispatch it starts from
  int32_t *counts_all, *offsets_all, *src_all, *pos_all;
  // MXFP8 activations (W4A8): input codes and scales of the up products
  // (x_q: the model-width rows; xl_q: the latent rows of a latent layer),
  // the ReLU^2 output's scales ([j][packed row], [j][token]); the ReLU^2
  // codes reuse h / h_s
  uint8_t *x_q, *xl_q, *xs_r, *xs_s, *hs_r, *hs_s;
  uint8_t* xs_t;  // the routed product's input scales in token order ([j][token]; xs_s when that is the same)
  long ldT, ldR;
  // decode path
  int32_t *items, *n_items;
  int ncr, ncs, max_items;
  float *part, *part_s;
  PlanSpec up, down;
};

size_t carve_forward(const moe_layer_desc* d, int T, void* ws, FwdBufs* b) {
  Carver c(ws);
  const int E = d->E, K = d->K, F = d->F, Fs = d->F_shared, L = d->d_latent;
  const int de = L ? L : d->d;
  const long R = (long)T * K;
  const size_t as = act_size(d->act_dtype);
  const int Tc = T > 0 ? T : 1;
  b->decode = decode_path(d, T);
  if (d->act_dtype == MOE_BF16 && !b->decode) {
    b->S = router_bf16_splits(Tc, d->d, E);
    b->w3 = c.take<uint16_t>((size_t)E * 3 * router_plane_width(d->d));
    b->logits = c.take<float>((size_t)b->S * Tc * E);
  } else {
    b->S = 1;
    b->w3 = nullptr;
    b->logits = c.take<float>((size_t)Tc * E);
  }
  b->ids = c.take<int32_t>((size_t)Tc * K);
  b->wts = c.take<float>((size_t)Tc * K);
  b->counts = c.take<int32_t>(E);
  b->offsets = c.take<int32_t>(E + 1);
  b->route_src = c.take<int32_t>(R > 0 ? R : 1);
  b->route_pos = c.take<int32_t>(R > 0 ? R : 1);
  if (d->capacity_factor > 0.0f && !b->decode) {
    b->counts_all = c.take<int32_t>(E);
    b->offsets_all = c.take<int32_t>(E + 1);
    b->src_all = c.take<int32_t>(R > 0 ? R : 1);
    b->pos_all = c.take<int32_t>(R > 0 ? R : 1);
  } else {
    b->counts_all = b->offsets_all = b->src_all = b->pos_all = nullptr;
  }
  b->x_norm = (d->flags & MOE_FLAG_PRENORM_RESIDUAL) ? c.take<char>((size_t)Tc * d->d * as) : nullptr;
  b->x_q = b->xl_q = b->xs_r = b->xs_s = b->hs_r = b->hs_s = b->xs_t = nullptr;
  b->ldT = mx_scale_ld(Tc);
  b->ldR = mx_scale_ld(R > 0 ? R : 1);
  if ((d->flags & MOE_FLAG_MXFP8_ACTIVATIONS) && !b->decode) {
    if (!L || Fs) b->x_q = c.take<uint8_t>((size_t)Tc * d->d);
    if (L) b->xl_q = c.take<uint8_t>((size_t)Tc * L);
    b->xs_r = c.take<uint8_t>((size_t)(de / kMxBlock) * b->ldR);
    b->hs_r = c.take<uint8_t>((size_t)(F / kMxBlock) * b->ldR);
    if (Fs) {
      b->xs_s = c.take<uint8_t>((size_t)(d->d / kMxBlock) * b->ldT);
      b->hs_s = c.take<uint8_t>((size_t)(Fs / kMxBlock) * b->ldT);
    }
    b->xs_t = (!L && Fs) ? b->xs_s : c.take<uint8_t>((size_t)(de / kMxBlock) * b->ldT);
  }
  b->x_lat = L ? c.take<char>((size_t)Tc * L * as) : nullptr;
  b->y_lat = L ? c.take<char>((size_t)Tc * L * as) : nullptr;
  b->y_s = Fs ? c.take<float>((size_t)Tc * d->d) : nullptr;
  b->S_lin = b->S_lout = 1;
  b->part_lat = nullptr;
  if (L && d->act_dtype == MOE_BF16) {
    b->S_lin = latent_splits(Tc, L, d->d);
    b->S_lout = latent_splits(Tc, d->d, L);
    const size_t n = std::max((size_t)b->S_lin * L, (size_t)b->S_lout * d->d) * Tc;
    if (b->S_lin > 1 || b->S_lout > 1) b->part_lat = c.take<float>(n);
  }
  if (b->decode) {
    b->ncr = ceil_div(F, kDecodeChunk);
    b->ncs = Fs ? ceil_div(Fs, kDecodeChunk) : 0;
    b->max_items = (int)decode_max_items(E, R, b->ncr, Fs ? T : 0, b->ncs);
    b->items = c.take<int32_t>(b->max_items > 0 ? b->max_items : 1);
    b->n_items = c.take<int32_t>(1);
    b->part = c.take<float>((size_t)(R > 0 ? R : 1) * b->ncr * de);
    b->part_s = Fs ? c.take<float>((size_t)Tc * b->ncs * d->d) : nullptr;
    b->dscratch = nullptr;
    b->plan_up = b->plan_down = b->num_tiles = nullptr;
    b->h = b->h_s = b->y_packed = nullptr;
    b->max_up = b->max_down = 0;
    return c.off + kAlign;
  }
  b->items = b->n_items = nullptr;
  b->part = b->part_s = nullptr;
  b->ncr = b->ncs = b->max_items = 0;
  b->dscratch = c.take<char>(dispatch_scratch_bytes(Tc, E));
  b->up = PlanSpec{E, Fs ? T : 0, ceil_div(F, kTileN), ceil_div(Fs > 0 ? Fs : 1, kTileN)};
  b->down = PlanSpec{E, Fs ? T : 0, ceil_div(de, kTileN), ceil_div(d->d, kTileN)};
  b->max_up = plan_max_tiles(b->up, R);
  b->max_down = plan_max_tiles(b->down, R);
  b->plan_up = c.take<int32_t>(2 * (size_t)b->max_up + 2);
  b->plan_down = c.take<int32_t>(2 * (size_t)b->max_down + 2);
  b->num_tiles = c.take<int32_t>(2);
  b->h = c.take<char>((size_t)(R > 0 ? R : 1) * F * as);
  b->h_s = Fs ? c.take<char>((size_t)Tc * Fs * as) : nullptr;
  b->y_packed = c.take<char>((size_t)(R > 0 ? R : 1) * de * as);
  return c.off + kAlign;
}

moe_status check_desc(const moe_layer_desc* d, int T) {
  if (!d) return MOE_ERR_INVALID_ARG;
  moe_status st = check_router(T, d->E, d->K, d->n_group, d->topk_group);
  if (st != MOE_OK) return st;
  if (d->d < 1 || d->F < 1 || d->F_shared < 0 || d->d_latent < 0) return MOE_ERR_INVALID_ARG;
  if (d->act_dtype != MOE_F32 && d->act_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (d->flags & ~(MOE_FLAG_ZERO_SKIP_DOWN | MOE_FLAG_ACCUMULATE_OUT | MOE_FLAG_PRENORM_RESIDUAL |
                   MOE_FLAG_FP8_EXPERTS | MOE_FLAG_MXFP4_EXPERTS | MOE_FLAG_MXFP8_ACTIVATIONS))
    return MOE_ERR_INVALID_ARG;
  if ((d->flags & MOE_FLAG_MXFP8_ACTIVATIONS) && !(d->flags & MOE_FLAG_MXFP4_EXPERTS)) return MOE_ERR_INVALID_ARG;
  if ((d->flags & MOE_FLAG_FP8_EXPERTS) && (d->flags & MOE_FLAG_MXFP4_EXPERTS)) return MOE_ERR_INVALID_ARG;
  if ((d->flags & MOE_FLAG_ACCUMULATE_OUT) && (d->flags & MOE_FLAG_PRENORM_RESIDUAL)) return MOE_ERR_INVALID_ARG;
  if ((d->flags & MOE_FLAG_PRENORM_RESIDUAL) && !(d->norm_eps >= 0.0f && d->norm_eps < INFINITY))
    return MOE_ERR_INVALID_ARG;
  if (!(d->capacity_factor >= 0.0f && d->capacity_factor < INFINITY)) return MOE_ERR_INVALID_ARG;
  if (d->capacity_factor > 0.0f && capacity_slots(T > 0 ? T : 1, d->K, d->E, d->capacity_factor) < 0)
    return MOE_ERR_UNSUPPORTED;
  if (d->d % 8 || d->F % 8 || d->F_shared % 8 || d->d_latent % 8) return MOE_ERR_UNSUPPORTED;
  if (d->flags & MOE_FLAG_FP8_EXPERTS) {
    if (d->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (d->d % 16 || d->F % 16 || d->F_shared % 16 || d->d_latent % 16) return MOE_ERR_UNSUPPORTED;
  }
  if (d->flags & MOE_FLAG_MXFP4_EXPERTS) {
    if (d->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (d->d % kMxBlock || d->F % kMxBlock || d->F_shared % kMxBlock || d->d_latent % kMxBlock)
      return MOE_ERR_UNSUPPORTED;
  }
  if (d->d > kMaxWidth || d->d_latent > kMaxWidth) return MOE_ERR_UNSUPPORTED;
  {
    const long as = (long)act_size(d->act_dtype), R = (long)T * d->K;
    const long de = d->d_latent ? d->d_latent : d->d;
    if (!fits_operand(T, d->d, as) || !fits_operand(T, d->d_latent, as) || !fits_operand(R, d->F, as) ||
        !fits_operand(R, de, as) || !fits_operand(T, d->F_shared, as) ||
        (d->F_shared && !fits_operand(T, d->d, 4)))
      return MOE_ERR_UNSUPPORTED;
    if ((long)d->F * de * as > kMaxWeightBytes || (long)d->F_shared * d->d * as > kMaxWeightBytes ||
        (long)d->d_latent * d->d * as > kMaxWeightBytes)
      return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: an argument breaks the layer's constraints";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: valid for the layer, outside this library's limits";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: the HIP runtime reported an error";
  }
  return "unknown moe_status";
}

// ---------------------------------------------------------------------------
moe_status moe_pack_weight(const void* src, moe_dtype dt, int G, int R, int C, int kind, void* dst,
                           moe_stream_t stream) {
  if (G < 0 || R < 0 || C < 0) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16 && dt != MOE_FP8_E4M3 && dt != MOE_MXFP4) return MOE_ERR_INVALID_ARG;
  if (kind != MOE_PACK_OUT_IN && kind != MOE_PACK_NEURON_MAJOR) return MOE_ERR_INVALID_ARG;
  if (C % (dt == MOE_MXFP4 ? 32 : dt == MOE_FP8_E4M3 ? 16 : 8)) return MOE_ERR_UNSUPPORTED;
  // bytes per two elements (MXFP4 codes are half a byte)
  const size_t eb2 = dt == MOE_MXFP4 ? 1 : dt == MOE_FP8_E4M3 ? 2 : dt == MOE_BF16 ? 4 : 8;
  if ((size_t)R * C * eb2 / 2 > (size_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if ((long)G * R * C == 0) return MOE_OK;
  if (!src || !dst) return MOE_ERR_INVALID_ARG;
  const size_t bytes = (size_t)G * R * C * eb2 / 2;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return MOE_ERR_INVALID_ARG;
  if (!aligned16(src) || !aligned16(dst)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_pack_weight(src, (int)(eb2 / 2), kind == MOE_PACK_NEURON_MAJOR, G, R, C, dst,
                                       (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
moe_status moe_quantize_fp8(const void* w, moe_dtype dt, long rows, int C, uint8_t* codes, float* scales,
                            moe_stream_t stream) {
  if (rows < 0 || C < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!w || !codes || !scales) return MOE_ERR_INVALID_ARG;
  if (rows > (long)INT_MAX * 4) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_quantize_fp8(w, dt == MOE_BF16, rows, C, codes, scales, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
moe_status moe_quantize_mxfp4(const void* w, moe_dtype dt, int G, int R, int C, uint8_t* codes, uint8_t* scales,
                              moe_stream_t stream) {
  if (G < 0 || R < 0 || C < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (C % kMxBlock) return MOE_ERR_UNSUPPORTED;
  if ((long)G * R == 0) return MOE_OK;
  if (!w || !codes || !scales) return MOE_ERR_INVALID_ARG;
  if ((long)R * C > INT_MAX) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(w) || !aligned16(codes)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_quantize_mxfp4(w, dt == MOE_BF16, G, R, C, codes, scales, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
moe_status moe_quantize_mxfp8(const void* x, moe_dtype dt, int rows, int C, uint8_t* codes, uint8_t* scales, long ld,
                              moe_stream_t stream) {
  if (rows < 0 || C < 1 || ld < rows) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (C % kMxBlock) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!x || !codes || !scales) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(codes)) return MOE_ERR_UNSUPPORTED;
  if ((long)rows * C * 2 >= kMaxOperandBytes) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_quantize_act_mxfp8((const uint16_t*)x, rows, C, codes, scales, ld, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
moe_status moe_rmsnorm(const void* x, const void* w_norm, float eps, int T, int d, moe_dtype dt, void* out,
                       moe_stream_t stream) {
  if (T < 0 || d < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (!(eps >= 0.0f && eps < INFINITY)) return MOE_ERR_INVALID_ARG;
  if (d % 8 || d > kMaxWidth) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_norm || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_norm) || !aligned16(out)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_rmsnorm(x, w_norm, eps, T, d, dt == MOE_BF16, out, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
size_t moe_router_logits_workspace_size(int T, int d, int E, moe_dtype dt) {
  if (T <= 0 || d <= 0 || E <= 0 || dt != MOE_BF16) return 0;
  const int S = router_bf16_splits(T, d, E);
  Carver c(nullptr);
  c.take<uint16_t>((size_t)E * 3 * router_plane_width(d));
  c.take<float>((size_t)S * T * E);
  return c.off + kAlign;
}

moe_status moe_router_logits(const void* x, moe_dtype dt, int T, int d, const float* w_router,
                             int E, float* logits, void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (T < 0 || d < 1 || E < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || d % 8) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !logits) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x)) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  if (dt == MOE_F32) return hip_status(launch_router_gemm_f32(x, 0, T, d, w_router, E, logits, s));
  const size_t need = moe_router_logits_workspace_size(T, d, E, dt);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  const int S = router_bf16_splits(T, d, E);
  Carver c(ws);
  uint16_t* w3 = c.take<uint16_t>((size_t)E * 3 * router_plane_width(d));
  float* part = c.take<float>((size_t)S * T * E);
  MOE_TRY(launch_split_router_weight(w_router, E, d, w3, s));
  MOE_TRY(launch_router_gemm_bf16x3((const uint16_t*)x, T, d, w3, E, part, S, s));
  return hip_status(launch_sum_partials(part, S, (long)T * E, logits, s));
}

// ---------------------------------------------------------------------------
moe_status moe_route(const float* logits, const float* bias, int T, int E, int K, int n_group,
                     int topk_group, int norm_topk_prob, float routed_scaling_factor, int32_t* ids,
                     float* weights, moe_stream_t stream) {
  const moe_status st = check_router(T, E, K, n_group, topk_group);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!logits || !ids || !weights) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_route(logits, 1, bias, T, E, K, n_group, topk_group, norm_topk_prob ? 1 : 0,
                                 routed_scaling_factor, ids, weights, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
size_t moe_dispatch_workspace_size(int T, int K, int E) {
  (void)K;
  if (T <= 0 || E <= 0) return 0;
  return dispatch_scratch_bytes(T, E) + kAlign;
}

moe_status moe_dispatch(const int32_t* ids, int T, int K, int E, int32_t* counts, int32_t* offsets,
                        int32_t* route_src, int32_t* route_pos, void* ws, size_t ws_bytes,
                        moe_stream_t stream) {
  if (T < 0 || K < 1 || E < 1 || K > E) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || K > MOE_MAX_TOPK || (long)T * K > kMaxRoutes) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!ids || !counts || !offsets || !route_src || !route_pos) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < moe_dispatch_workspace_size(T, K, E)) return MOE_ERR_WORKSPACE;
  return hip_status(launch_dispatch(ids, T, K, E, counts, offsets, route_src, route_pos, ws, nullptr,
                                    (hipStream_t)stream));
}

int moe_capacity_slots(int T, int K, int E, float capacity_factor) {
  if (T < 0 || K < 1 || E < 1 || !(capacity_factor >= 0.0f && capacity_factor < INFINITY)) return -1;
  return (int)capacity_slots(T, K, E, capacity_factor);
}

size_t moe_dispatch_capacity_workspace_size(int T, int K, int E) {
  if (T <= 0 || E <= 0 || K <= 0) return 0;
  Carver c(nullptr);
  c.take<char>(dispatch_scratch_bytes(T, E));
  c.take<int32_t>(E);
  c.take<int32_t>(E + 1);
  c.take<int32_t>((size_t)T * K);
  c.take<int32_t>((size_t)T * K);
  return c.off + kAlign;
}

moe_status moe_dispatch_capacity(const int32_t* ids, const float* weights, int T, int K, int E, int capacity,
                                 int32_t* counts, int32_t* offsets, int32_t* route_src, int32_t* route_pos,
                                 void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (T < 0 || K < 1 || E < 1 || K > E || capacity < 0) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || K > MOE_MAX_TOPK || (long)T * K > kMaxRoutes) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!ids || !weights || !counts || !offsets || !route_src || !route_pos) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < moe_dispatch_capacity_workspace_size(T, K, E)) return MOE_ERR_WORKSPACE;
  Carver c(ws);
  void* scratch = c.take<char>(dispatch_scratch_bytes(T, E));
  int32_t* counts_all = c.take<int32_t>(E);
  int32_t* offsets_all = c.take<int32_t>(E + 1);
  int32_t* src_all = c.take<int32_t>((size_t)T * K);
  int32_t* pos_all = c.take<int32_t>((size_t)T * K);
  hipStream_t s = (hipStream_t)stream;
  MOE_TRY(launch_dispatch(ids, T, K, E, counts_all, offsets_all, src_all, pos_all, scratch, nullptr, s));
  return hip_status(launch_capacity(counts_all, offsets_all, src_all, weights, E, capacity, counts, offsets,
                                    route_src, route_pos, s));
}

// ---------------------------------------------------------------------------
namespace {
// Whether the staged expert call runs the decode path (live-neuron skipping).
bool experts_decode(moe_dtype dt, int T, int d_e, int F, int flags) {
  return (flags & MOE_FLAG_ZERO_SKIP_DOWN) && dt == MOE_BF16 && T <= kDecodeMaxRows && d_e <= kDecodeMaxWidth &&
         ceil_div(F, kDecodeChunk) <= kMaxDecodeChunks;
}
struct ExpBufs {
  bool decode;
  int32_t *plan_up, *plan_down, *num_tiles;
  void* h;
  PlanSpec up, down;
  long max_up, max_down;
  int32_t *items, *n_items;
  float* part;
  int ncr, max_items;
};
size_t carve_experts(moe_dtype dt, int T, int d_e, int K, int E, int F, int flags, void* ws, ExpBufs* b) {
  Carver c(ws);
  const long R = (long)T * K;
  b->decode = experts_decode(dt, T, d_e, F, flags);
  if (b->decode) {
    b->ncr = ceil_div(F, kDecodeChunk);
    b->max_items = (int)decode_max_items(E, R, b->ncr, 0, 0);
    b->items = c.take<int32_t>(b->max_items > 0 ? b->max_items : 1);
    b->n_items = c.take<int32_t>(1);
    b->part = c.take<float>((size_t)(R > 0 ? R : 1) * b->ncr * d_e);
    b->plan_up = b->plan_down = b->num_tiles = nullptr;
    b->h = nullptr;
    b->max_up = b->max_down = 0;
    return c.off + kAlign;
  }
  b->items = b->n_items = nullptr;
  b->part = nullptr;
  b->ncr = b->max_items = 0;
  b->up = PlanSpec{E, 0, ceil_div(F, kTileN), 1};
  b->down = PlanSpec{E, 0, ceil_div(d_e, kTileN), 1};
  b->max_up = plan_max_tiles(b->up, R);
  b->max_down = plan_max_tiles(b->down, R);
  b->plan_up = c.take<int32_t>(2 * (size_t)b->max_up + 2);
  b->plan_down = c.take<int32_t>(2 * (size_t)b->max_down + 2);
  b->num_tiles = c.take<int32_t>(2);
  b->h = c.take<char>((size_t)(R > 0 ? R : 1) * F * act_size(dt));
  return c.off + kAlign;
}
}  // namespace

size_t moe_experts_workspace_size(moe_dtype dt, int T, int d_e, int K, int E, int F, int flags) {
  if (T < 0 || d_e < 1 || K < 1 || E < 1 || F < 1) return 0;
  ExpBufs b;
  return carve_experts(dt, T, d_e, K, E, F, flags, nullptr, &b);
}

namespace {
// The low-precision expert weights of moe_experts_fp8 / moe_experts_mxfp4.
struct ExpQuant {
  bool w8 = false, w4 = false;
  const float *s_up = nullptr, *s_dn = nullptr;   // FP8 scales
  const void* w_down = nullptr;                   // MXFP4: down codes packed [OUT_IN]
  const uint8_t *e_up = nullptr, *e_dn = nullptr; // MXFP4 scales
};

// moe_experts, moe_experts_fp8 and moe_experts_mxfp4.
moe_status experts_impl(const void* x, moe_dtype dt, int T, int d_e, int K, const int32_t* route_src,
                        const int32_t* offsets, int E, int F, const void* w_up, const void* w_down_t,
                        const ExpQuant& qz, int flags, void* y_packed, int64_t* zero_count, void* ws,
                        size_t ws_bytes, moe_stream_t stream) {
  const bool w8 = qz.w8, w4 = qz.w4;
  const float *s_up = qz.s_up, *s_dn = qz.s_dn;
  if (T < 0 || K < 1 || E < 1 || F < 1 || d_e < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if ((w8 || w4) && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (flags & ~MOE_FLAG_ZERO_SKIP_DOWN) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || (long)T * K > kMaxRoutes) return MOE_ERR_UNSUPPORTED;
  if (d_e % 8 || F % 8) return MOE_ERR_UNSUPPORTED;
  if (w8 && (d_e % 16 || F % 16)) return MOE_ERR_UNSUPPORTED;
  if (w4 && (d_e % kMxBlock || F % kMxBlock)) return MOE_ERR_UNSUPPORTED;
  {
    const long as = (long)act_size(dt), R = (long)T * K;
    if (!fits_operand(T, d_e, as) || !fits_operand(R, F, as) || !fits_operand(R, d_e, as))
      return MOE_ERR_UNSUPPORTED;
    if ((long)F * d_e * as > kMaxWeightBytes) return MOE_ERR_UNSUPPORTED;
  }
  if (zero_count && !experts_decode(dt, T, d_e, F, flags)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !offsets || !w_up || !w_down_t || !y_packed) return MOE_ERR_INVALID_ARG;
  if (w8 && (!s_up || !s_dn)) return MOE_ERR_INVALID_ARG;
  if (w4 && (!qz.w_down || !qz.e_up || !qz.e_dn)) return MOE_ERR_INVALID_ARG;
  if (w4 && !aligned16(qz.w_down)) return MOE_ERR_UNSUPPORTED;
  if (!route_src && K != 1) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_up) || !aligned16(w_down_t) || !aligned16(y_packed))
    return MOE_ERR_UNSUPPORTED;
  if (w8 && (!aligned16(s_up) || !aligned16(s_dn))) return MOE_ERR_UNSUPPORTED;
  ExpBufs b;
  const size_t need = carve_experts(dt, T, d_e, K, E, F, flags, nullptr, &b);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  carve_experts(dt, T, d_e, K, E, F, flags, ws, &b);
  hipStream_t s = (hipStream_t)stream;
  const int bf = dt == MOE_BF16;
  const long R = (long)T * K;

  if (b.decode) {
    MOE_TRY(launch_decode_items(offsets, E, b.ncr, b.items, b.n_items, s));
    DecodeArgs a = {};
    a.E = E;
    a.K = K;
    a.offsets = offsets;
    a.route_src = route_src;
    a.x = (const uint16_t*)x;
    a.ldx = d_e;
    a.d_e = d_e;
    a.F = F;
    a.w_up = w_up;
    a.w_dn = w_down_t;
    a.w8 = w8;
    a.s_up = s_up;
    a.s_dn = s_dn;
    a.w4 = w4;
    a.e_up = qz.e_up;
    a.e_dn = qz.e_dn;
    a.part = b.part;
    a.ncr = b.ncr;
    a.items = b.items;
    a.n_items = b.n_items;
    a.zero_count = (unsigned long long*)zero_count;
    MOE_TRY(launch_expert_decode(a, b.max_items, s));
    return hip_status(launch_reduce_chunks(b.part, (int)R, b.ncr, d_e, y_packed, 1, nullptr, 0, 0, 0, nullptr, s));
  }

  PlanOut P{b.plan_up, b.plan_down, b.num_tiles, b.up, b.down};
  MOE_TRY(launch_plan(offsets, &P, s));

  GemmArgs up = {};
  up.E = E;
  up.offsets = offsets;
  up.gather = route_src;
  up.gdiv = K;
  up.A = x;
  up.lda = d_e;
  up.B = w_up;
  up.strideB = (long)F * d_e;
  up.ldb = d_e;
  up.b_packed = 1;
  up.b_fp8 = w8;
  up.bscale = s_up;
  up.b_fp4 = w4;
  up.e8 = qz.e_up;
  up.N = F;
  up.Kd = d_e;
  up.C = b.h;
  up.ldc = F;
  up.c_f32 = !bf;
  up.plan = b.plan_up;
  up.num_tiles = b.num_tiles;
  up.ksplit = 1;
  MOE_TRY(launch_gemm(up, bf, B_NK, EPI_RELU2, (int)b.max_up, s));

  GemmArgs dn = {};
  dn.E = E;
  dn.offsets = offsets;
  dn.A = b.h;
  dn.lda = F;
  // MXFP4: the [OUT_IN] copy of the down codes, read like the up weights
  dn.B = w4 ? qz.w_down : w_down_t;
  dn.strideB = (long)F * d_e;
  dn.ldb = w4 ? F : d_e;
  dn.b_packed = 1;
  dn.b_fp8 = w8;
  dn.bscale = s_dn;
  dn.b_fp4 = w4;
  dn.e8 = qz.e_dn;
  dn.N = d_e;
  dn.Kd = F;
  dn.C = y_packed;
  dn.ldc = d_e;
  dn.c_f32 = !bf;
  dn.plan = b.plan_down;
  dn.num_tiles = b.num_tiles + 1;
  dn.ksplit = 1;
  return hip_status(launch_gemm(dn, bf, w4 ? B_NK : B_KN, EPI_STORE, (int)b.max_down, s));
}
}  // namespace

moe_status moe_experts(const void* x, moe_dtype dt, int T, int d_e, int K, const int32_t* route_src,
                       const int32_t* offsets, int E, int F, const void* w_up, const void* w_down_t,
                       int flags, void* y_packed, int64_t* zero_count, void* ws, size_t ws_bytes,
                       moe_stream_t stream) {
  return experts_impl(x, dt, T, d_e, K, route_src, offsets, E, F, w_up, w_down_t, ExpQuant{}, flags, y_packed,
                      zero_count, ws, ws_bytes, stream);
}

moe_status moe_experts_fp8(const void* x, moe_dtype dt, int T, int d_e, int K, const int32_t* route_src,
                           const int32_t* offsets, int E, int F, const void* w_up, const float* w_up_scale,
                           const void* w_down_t, const float* w_down_scale, int flags, void* y_packed,
                           int64_t* zero_count, void* ws, size_t ws_bytes, moe_stream_t stream) {
  ExpQuant qz;
  qz.w8 = true;
  qz.s_up = w_up_scale;
  qz.s_dn = w_down_scale;
  return experts_impl(x, dt, T, d_e, K, route_src, offsets, E, F, w_up, w_down_t, qz, flags, y_packed, zero_count,
                      ws, ws_bytes, stream);
}

moe_status moe_experts_mxfp4(const void* x, moe_dtype dt, int T, int d_e, int K, const int32_t* route_src,
                             const int32_t* offsets, int E, int F, const void* w_up, const uint8_t* w_up_e8,
                             const void* w_down_t, const void* w_down, const uint8_t* w_down_e8, int flags,
                             void* y_packed, int64_t* zero_count, void* ws, size_t ws_bytes, moe_stream_t stream) {
  ExpQuant qz;
  qz.w4 = true;
  qz.w_down = w_down;
  qz.e_up = w_up_e8;
  qz.e_dn = w_down_e8;
  return experts_impl(x, dt, T, d_e, K, route_src, offsets, E, F, w_up, w_down_t, qz, flags, y_packed, zero_count,
                      ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
moe_status moe_combine(const void* y_packed, const float* weights, const int32_t* ids,
                       const int32_t* route_pos, const float* y_shared, int T, int K, int d,
                       moe_dtype dt, int flags, void* out, moe_stream_t stream) {
  if (T < 0 || K < 1 || d < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (flags & ~(MOE_FLAG_ACCUMULATE_OUT | MOE_FLAG_ZERO_SKIP_DOWN)) return MOE_ERR_INVALID_ARG;
  if (d % 8 || d > kMaxWidth || K > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (!fits_operand((long)T * K, d, act_size(dt)) || !fits_operand(T, d, act_size(dt)) ||
      (y_shared && !fits_operand(T, d, 4)))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y_packed || !weights || !ids || !route_pos || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y_packed) || !aligned16(out) || (y_shared && !aligned16(y_shared))) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_combine(y_packed, dt == MOE_BF16, weights, ids, route_pos, y_shared, T, K, d,
                                   (flags & MOE_FLAG_ACCUMULATE_OUT) ? out : nullptr, out, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
size_t moe_workspace_size(const moe_layer_desc* desc, int T) {
  if (check_desc(desc, T) != MOE_OK) return 0;
  FwdBufs b;
  return carve_forward(desc, T, nullptr, &b);
}

moe_status moe_workspace_routing(const moe_layer_desc* desc, int T, moe_routing_layout* out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  const moe_status st = check_desc(desc, T);
  if (st != MOE_OK) return st;
  // carve against a stand-in base address (never dereferenced) to read the
  // offsets of the routing buffers
  char* const base = (char*)(uintptr_t)(1u << 20);
  FwdBufs b;
  carve_forward(desc, T, base, &b);
  out->ids = (size_t)((char*)b.ids - base);
  out->weights = (size_t)((char*)b.wts - base);
  out->counts = (size_t)((char*)b.counts - base);
  out->offsets = (size_t)((char*)b.offsets - base);
  out->route_src = (size_t)((char*)b.route_src - base);
  out->route_pos = (size_t)((char*)b.route_pos - base);
  return MOE_OK;
}

moe_status moe_layer_forward_timed(const moe_layer_desc* desc, const moe_layer_weights* w,
                                   const void* x_in, int T, void* out, void* ws, size_t ws_bytes,
                                   moe_stream_t stream, void* const* events) {
  moe_status st = check_desc(desc, T);
  if (st != MOE_OK) return st;
  if (!w) return MOE_ERR_INVALID_ARG;
  const moe_layer_desc& d = *desc;
  if (!w->w_router || !w->w_up || !w->w_down_t) return MOE_ERR_INVALID_ARG;
  if (d.F_shared && (!w->w_up_shared || !w->w_down_shared_t)) return MOE_ERR_INVALID_ARG;
  if (d.d_latent && (!w->w_latent_in || !w->w_latent_out)) return MOE_ERR_INVALID_ARG;
  const bool prenorm = (d.flags & MOE_FLAG_PRENORM_RESIDUAL) != 0;
  if (prenorm && !w->w_norm) return MOE_ERR_INVALID_ARG;
  const bool w8 = (d.flags & MOE_FLAG_FP8_EXPERTS) != 0;
  if (w8 && (!w->w_up_scale || !w->w_down_scale)) return MOE_ERR_INVALID_ARG;
  if (w8 && d.F_shared && (!w->w_up_shared_scale || !w->w_down_shared_scale)) return MOE_ERR_INVALID_ARG;
  const bool w4 = (d.flags & MOE_FLAG_MXFP4_EXPERTS) != 0;
  const bool mx8 = (d.flags & MOE_FLAG_MXFP8_ACTIVATIONS) != 0 && !decode_path(desc, T);
  if (w4 && (!w->w_down || !w->w_up_e8 || !w->w_down_e8)) return MOE_ERR_INVALID_ARG;
  if (w4 && d.F_shared && (!w->w_down_shared || !w->w_up_shared_e8 || !w->w_down_shared_e8))
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x_in || !out) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {x_in, out, w->w_up, w->w_down_t, w->w_up_shared, w->w_down_shared_t,
                        w->w_latent_in, w->w_latent_out, w->w_norm,
                        w4 ? w->w_down : nullptr, w4 ? w->w_down_shared : nullptr};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_UNSUPPORTED;
  if (w8) {
    const void* sp[] = {w->w_up_scale, w->w_down_scale, w->w_up_shared_scale, w->w_down_shared_scale};
    for (const void* p : sp)
      if (p && !aligned16(p)) return MOE_ERR_UNSUPPORTED;
  }
  FwdBufs b;
  const size_t need = carve_forward(desc, T, nullptr, &b);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  carve_forward(desc, T, ws, &b);

  hipStream_t s = (hipStream_t)stream;
  auto rec = [&](int i) -> hipError_t {
    return events ? hipEventRecord((hipEvent_t)events[i], s) : hipSuccess;
  };
  const int bf = d.act_dtype == MOE_BF16;
  const int E = d.E, K = d.K, F = d.F, Fs = d.F_shared, L = d.d_latent;
  const int de = L ? L : d.d;
  const size_t as = act_size(d.act_dtype);

  // with the fused front and back, the layer runs on RMSNorm(x_in) and x_in
  // joins the final fp32 sum as the residual; otherwise the old output does
  // when accumulating
  MOE_TRY(rec(2 * MOE_STAGE_NORM));
  const void* x = x_in;
  if (prenorm) {
    MOE_TRY(launch_rmsnorm(x_in, w->w_norm, d.norm_eps, T, d.d, bf, b.x_norm, s));
    x = b.x_norm;
  }
  MOE_TRY(rec(2 * MOE_STAGE_NORM + 1));
  const void* resid = prenorm ? x_in : ((d.flags & MOE_FLAG_ACCUMULATE_OUT) ? out : nullptr);

  // router logits (fp32)
  MOE_TRY(rec(2 * MOE_STAGE_ROUTER_GEMM));
  if (b.decode) {
    MOE_TRY(launch_router_small((const uint16_t*)x, T, d.d, w->w_router, E, b.logits, s));
  } else if (bf) {
    MOE_TRY(launch_split_router_weight(w->w_router, E, d.d, b.w3, s));
    MOE_TRY(launch_router_gemm_bf16x3((const uint16_t*)x, T, d.d, b.w3, E, b.logits, b.S, s));
  } else {
    MOE_TRY(launch_router_gemm_f32(x, 0, T, d.d, w->w_router, E, b.logits, s));
  }
  MOE_TRY(rec(2 * MOE_STAGE_ROUTER_GEMM + 1));

  // small decode batches route and dispatch inside the expert kernel
  const bool fused = b.decode && T >= 1 && T <= kFusedRows && E <= kFusedExperts;
  MOE_TRY(rec(2 * MOE_STAGE_ROUTE));
  if (!fused)
    MOE_TRY(launch_route(b.logits, b.S, w->bias, T, E, K, d.n_group, d.topk_group, d.norm_topk_prob ? 1 : 0,
                         d.routed_scaling_factor, b.ids, b.wts, s));
  MOE_TRY(rec(2 * MOE_STAGE_ROUTE + 1));

  MOE_TRY(rec(2 * MOE_STAGE_DISPATCH));
  PlanOut P{b.plan_up, b.plan_down, b.num_tiles, b.up, b.down};
  if (fused) {
    // nothing: the expert kernel dispatches
  } else if (b.decode)
    MOE_TRY(launch_dispatch_small(b.ids, T, K, E, b.counts, b.offsets, b.route_src, b.route_pos, b.ncr,
                                  b.ncs, b.items, b.n_items, s));
  else if (b.counts_all) {
    // capacity-bounded: dispatch every route, keep each expert's first C by
    // (gate, token, slot), then the tile plans of the accepted rows
    const int C = (int)capacity_slots(T, K, E, d.capacity_factor);
    MOE_TRY(launch_dispatch(b.ids, T, K, E, b.counts_all, b.offsets_all, b.src_all, b.pos_all, b.dscratch,
                            nullptr, s));
    MOE_TRY(launch_capacity(b.counts_all, b.offsets_all, b.src_all, b.wts, E, C, b.counts, b.offsets,
                            b.route_src, b.route_pos, s));
    MOE_TRY(launch_plan(b.offsets, &P, s));
  } else
    MOE_TRY(launch_dispatch(b.ids, T, K, E, b.counts, b.offsets, b.route_src, b.route_pos, b.dscratch, &P, s));
  MOE_TRY(rec(2 * MOE_STAGE_DISPATCH + 1));

  MOE_TRY(rec(2 * MOE_STAGE_LATENT_IN));
  if (L) {
    GemmArgs li = {};
    li.M_s = T;
    li.A_s = x;
    li.lda_s = d.d;
    li.B_s = w->w_latent_in;
    li.ldb_s = d.d;
    li.b_packed = 1;
    li.N_s = L;
    li.Kd_s = d.d;
    li.C_s = b.x_lat;
    li.ldc_s = L;
    li.c_s_f32 = !bf;
    li.ksplit = 1;
    if (bf && b.S_lin > 1) {
      // split over K into fp32 partials, summed and rounded once
      li.split_main = 1;
      li.ksplit = b.S_lin;
      li.C_s = b.part_lat;
      li.c_s_f32 = 1;
      li.split_stride = (long)T * L;
      MOE_TRY(launch_gemm(li, bf, B_NK, EPI_STORE, 0, s));
      MOE_TRY(launch_reduce_splits(b.part_lat, b.S_lin, (long)T * L, T, L, nullptr, 0, nullptr, b.x_lat, 1, s));
    } else {
      MOE_TRY(launch_gemm(li, bf, B_NK, EPI_STORE, 0, s));
    }
  }
  MOE_TRY(rec(2 * MOE_STAGE_LATENT_IN + 1));

  if (b.decode) {
    // up + ReLU^2 + live-neuron down for every (group, chunk) item in one
    // launch; the up stage records both stage events around it
    MOE_TRY(rec(2 * MOE_STAGE_UP));
    DecodeArgs a = {};
    a.E = E;
    a.K = K;
    a.offsets = b.offsets;
    a.route_src = b.route_src;
    a.x = (const uint16_t*)(L ? b.x_lat : x);
    a.ldx = de;
    a.d_e = de;
    a.F = F;
    a.w_up = w->w_up;
    a.w_dn = w->w_down_t;
    a.part = b.part;
    a.ncr = b.ncr;
    a.M_s = Fs ? T : 0;
    a.x_s = (const uint16_t*)x;
    a.ldx_s = d.d;
    a.d_s = d.d;
    a.F_s = Fs;
    a.w_up_s = w->w_up_shared;
    a.w_dn_s = w->w_down_shared_t;
    a.w8 = w8;
    if (w8) {
      a.s_up = w->w_up_scale;
      a.s_dn = w->w_down_scale;
      a.s_up_s = w->w_up_shared_scale;
      a.s_dn_s = w->w_down_shared_scale;
    }
    a.w4 = w4;
    if (w4) {
      a.e_up = w->w_up_e8;
      a.e_dn = w->w_down_e8;
      a.e_up_s = w->w_up_shared_e8;
      a.e_dn_s = w->w_down_shared_e8;
    }
    a.part_s = b.part_s;
    a.ncs = b.ncs;
    a.items = b.items;
    a.n_items = b.n_items;
    if (fused) {
      a.fused = 1;
      a.T = T;
      a.logits = b.logits;
      a.bias = w->bias;
      a.n_group = d.n_group;
      a.topk_group = d.topk_group;
      a.norm = d.norm_topk_prob ? 1 : 0;
      a.rsf = d.routed_scaling_factor;
      a.ids_out = b.ids;
      a.wts_out = b.wts;
      a.rpos_out = b.route_pos;
      a.counts_out = b.counts;
      a.offsets_out = b.offsets;
      a.src_out = b.route_src;
    }
    MOE_TRY(launch_expert_decode(a, b.max_items, s));
    MOE_TRY(rec(2 * MOE_STAGE_UP + 1));
    MOE_TRY(rec(2 * MOE_STAGE_DOWN));
    MOE_TRY(rec(2 * MOE_STAGE_DOWN + 1));
    MOE_TRY(rec(2 * MOE_STAGE_COMBINE));
    if (L) {
      // the shared rows' chunk partials -> y_s (fp32, added in the latent
      // projection's epilogue); the routes combined from their partials
      if (Fs) MOE_TRY(launch_reduce_chunks(b.part, 0, b.ncr, de, nullptr, 0, b.part_s, T, b.ncs, d.d, b.y_s, s));
      MOE_TRY(launch_combine_decode(b.part, b.ncr, b.wts, b.ids, b.route_pos, T, K, L, nullptr, 0, nullptr, b.y_lat,
                                    1, s));
    } else {
      MOE_TRY(launch_combine_decode(b.part, b.ncr, b.wts, b.ids, b.route_pos, T, K, d.d, Fs ? b.part_s : nullptr,
                                    b.ncs, resid, out, 1, s));
    }
    MOE_TRY(rec(2 * MOE_STAGE_COMBINE + 1));
  } else if (mx8) {
    // W4A8: the up products' inputs quantised to MXFP8 (codes, and scales in
    // packed-row order for the routed rows, token order for the shared
    // rows), then both projections on the block-scaled MFMA; the up
    // epilogue writes the ReLU^2 output as MXFP8 codes and scales
    MOE_TRY(rec(2 * MOE_STAGE_UP));
    if (L) {
      MOE_TRY(launch_quantize_act_mxfp8((const uint16_t*)b.x_lat, T, L, b.xl_q, b.xs_t, b.ldT, s));
      if (Fs) MOE_TRY(launch_quantize_act_mxfp8((const uint16_t*)x, T, d.d, b.x_q, b.xs_s, b.ldT, s));
    } else {
      MOE_TRY(launch_quantize_act_mxfp8((const uint16_t*)x, T, d.d, b.x_q, b.xs_t, b.ldT, s));
    }
    // the routed rows' scales in packed-row order (the accepted rows of a
    // capacity-bounded dispatch: offsets[E] of them)
    MOE_TRY(launch_gather_mx_scales(b.xs_t, b.ldT, b.route_src, b.offsets + E, K, de, T * K, b.xs_r, b.ldR, s));
    GemmArgs up = {};
    up.E = E;
    up.offsets = b.offsets;
    up.gather = b.route_src;
    up.gdiv = K;
    up.A = L ? b.xl_q : b.x_q;
    up.lda = de;
    up.as = b.xs_r;
    up.ld_as = b.ldR;
    up.B = w->w_up;
    up.strideB = (long)F * de;
    up.b_packed = 1;
    up.b_fp4 = 1;
    up.e8 = w->w_up_e8;
    up.N = F;
    up.Kd = de;
    up.C = b.h;
    up.ldc = F;
    up.cs = b.hs_r;
    up.ld_cs = b.ldR;
    up.M_s = Fs ? T : 0;
    up.A_s = b.x_q;
    up.lda_s = d.d;
    up.as_s = b.xs_s;
    up.ld_as_s = b.ldT;
    up.B_s = w->w_up_shared;
    up.e8_s = w->w_up_shared_e8;
    up.N_s = Fs;
    up.Kd_s = d.d;
    up.C_s = b.h_s;
    up.ldc_s = Fs;
    up.cs_s = b.hs_s;
    up.ld_cs_s = b.ldT;
    up.plan = b.plan_up;
    up.num_tiles = b.num_tiles;
    up.ksplit = 1;
    MOE_TRY(launch_gemm_mx(up, EPI_QRELU2, (int)b.max_up, s));
    MOE_TRY(rec(2 * MOE_STAGE_UP + 1));

    MOE_TRY(rec(2 * MOE_STAGE_DOWN));
    GemmArgs dn = {};
    dn.E = E;
    dn.offsets = b.offsets;
    dn.A = b.h;
    dn.lda = F;
    dn.as = b.hs_r;
    dn.ld_as = b.ldR;
    dn.B = w->w_down;  // the [OUT_IN] packing of the down codes
    dn.strideB = (long)F * de;
    dn.b_packed = 1;
    dn.b_fp4 = 1;
    dn.e8 = w->w_down_e8;
    dn.N = de;
    dn.Kd = F;
    dn.C = b.y_packed;
    dn.ldc = de;
    dn.c_f32 = 0;
    dn.M_s = Fs ? T : 0;
    dn.A_s = b.h_s;
    dn.lda_s = Fs;
    dn.as_s = b.hs_s;
    dn.ld_as_s = b.ldT;
    dn.B_s = w->w_down_shared;
    dn.e8_s = w->w_down_shared_e8;
    dn.N_s = d.d;
    dn.Kd_s = Fs;
    dn.C_s = b.y_s;
    dn.ldc_s = d.d;
    dn.c_s_f32 = 1;
    dn.plan = b.plan_down;
    dn.num_tiles = b.num_tiles + 1;
    dn.ksplit = 1;
    MOE_TRY(launch_gemm_mx(dn, EPI_STORE, (int)b.max_down, s));
    MOE_TRY(rec(2 * MOE_STAGE_DOWN + 1));

    MOE_TRY(rec(2 * MOE_STAGE_COMBINE));
    if (L)
      MOE_TRY(launch_combine(b.y_packed, bf, b.wts, b.ids, b.route_pos, nullptr, T, K, L, nullptr, b.y_lat, s));
    else
      MOE_TRY(launch_combine(b.y_packed, bf, b.wts, b.ids, b.route_pos, b.y_s, T, K, d.d, resid, out, s));
    MOE_TRY(rec(2 * MOE_STAGE_COMBINE + 1));
  } else {
    // routed + shared up projections with the ReLU^2 epilogue, one launch
    MOE_TRY(rec(2 * MOE_STAGE_UP));
    GemmArgs up = {};
    up.E = E;
    up.offsets = b.offsets;
    up.gather = b.route_src;
    up.gdiv = K;
    up.A = L ? b.x_lat : x;
    up.lda = de;
    up.B = w->w_up;
    up.strideB = (long)F * de;
    up.ldb = de;
    up.b_packed = 1;
    up.b_fp8 = w8;
    up.bscale = w8 ? w->w_up_scale : nullptr;
    up.bscale_s = w8 ? w->w_up_shared_scale : nullptr;
    up.b_fp4 = w4;
    up.e8 = w4 ? w->w_up_e8 : nullptr;
    up.e8_s = w4 ? w->w_up_shared_e8 : nullptr;
    up.N = F;
    up.Kd = de;
    up.C = b.h;
    up.ldc = F;
    up.c_f32 = !bf;
    up.M_s = Fs ? T : 0;
    up.A_s = x;
    up.lda_s = d.d;
    up.B_s = w->w_up_shared;
    up.ldb_s = d.d;
    up.N_s = Fs;
    up.Kd_s = d.d;
    up.C_s = b.h_s;
    up.ldc_s = Fs;
    up.c_s_f32 = !bf;
    up.plan = b.plan_up;
    up.num_tiles = b.num_tiles;
    up.ksplit = 1;
    MOE_TRY(launch_gemm(up, bf, B_NK, EPI_RELU2, (int)b.max_up, s));
    MOE_TRY(rec(2 * MOE_STAGE_UP + 1));

    // routed + shared down projections: y_packed in act dtype, y_s in fp32
    MOE_TRY(rec(2 * MOE_STAGE_DOWN));
    GemmArgs dn = {};
    dn.E = E;
    dn.offsets = b.offsets;
    dn.A = b.h;
    dn.lda = F;
    // MXFP4: the [OUT_IN] copies of the down codes, read like the up weights
    dn.B = w4 ? w->w_down : w->w_down_t;
    dn.strideB = (long)F * de;
    dn.ldb = w4 ? F : de;
    dn.b_packed = 1;
    dn.b_fp8 = w8;
    dn.bscale = w8 ? w->w_down_scale : nullptr;
    dn.bscale_s = w8 ? w->w_down_shared_scale : nullptr;
    dn.b_fp4 = w4;
    dn.e8 = w4 ? w->w_down_e8 : nullptr;
    dn.e8_s = w4 ? w->w_down_shared_e8 : nullptr;
    dn.N = de;
    dn.Kd = F;
    dn.C = b.y_packed;
    dn.ldc = de;
    dn.c_f32 = !bf;
    dn.M_s = Fs ? T : 0;
    dn.A_s = b.h_s;
    dn.lda_s = Fs;
    dn.B_s = w4 ? w->w_down_shared : w->w_down_shared_t;
    dn.ldb_s = w4 ? Fs : d.d;
    dn.N_s = d.d;
    dn.Kd_s = Fs;
    dn.C_s = b.y_s;
    dn.ldc_s = d.d;
    dn.c_s_f32 = 1;
    dn.plan = b.plan_down;
    dn.num_tiles = b.num_tiles + 1;
    dn.ksplit = 1;
    MOE_TRY(launch_gemm(dn, bf, w4 ? B_NK : B_KN, EPI_STORE, (int)b.max_down, s));
    MOE_TRY(rec(2 * MOE_STAGE_DOWN + 1));

    MOE_TRY(rec(2 * MOE_STAGE_COMBINE));
    if (L)
      MOE_TRY(launch_combine(b.y_packed, bf, b.wts, b.ids, b.route_pos, nullptr, T, K, L, nullptr, b.y_lat, s));
    else
      MOE_TRY(launch_combine(b.y_packed, bf, b.wts, b.ids, b.route_pos, b.y_s, T, K, d.d, resid, out, s));
    MOE_TRY(rec(2 * MOE_STAGE_COMBINE + 1));
  }

  MOE_TRY(rec(2 * MOE_STAGE_LATENT_OUT));
  if (L) {
    GemmArgs lo = {};
    lo.M_s = T;
    lo.A_s = b.y_lat;
    lo.lda_s = L;
    lo.B_s = w->w_latent_out;
    lo.ldb_s = L;
    lo.b_packed = 1;
    lo.N_s = d.d;
    lo.Kd_s = L;
    lo.C_s = out;
    lo.ldc_s = d.d;
    lo.c_s_f32 = !bf;
    lo.addend = b.y_s;
    lo.ld_add = d.d;
    lo.resid = resid;
    lo.ksplit = 1;
    if (bf && b.S_lout > 1) {
      // split over K into fp32 partials; the shared rows and the residual
      // source join in the reduction, before the one rounding
      lo.split_main = 1;
      lo.ksplit = b.S_lout;
      lo.C_s = b.part_lat;
      lo.c_s_f32 = 1;
      lo.split_stride = (long)T * d.d;
      lo.addend = nullptr;
      lo.resid = nullptr;
      MOE_TRY(launch_gemm(lo, bf, B_NK, EPI_STORE, 0, s));
      MOE_TRY(launch_reduce_splits(b.part_lat, b.S_lout, (long)T * d.d, T, d.d, b.y_s, d.d, resid, out, 1, s));
    } else {
      MOE_TRY(launch_gemm(lo, bf, B_NK, EPI_ADD_F32, 0, s));
    }
  }
  MOE_TRY(rec(2 * MOE_STAGE_LATENT_OUT + 1));
  (void)as;
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Backward pass
// ---------------------------------------------------------------------------
namespace {
struct BwdBufs {
  float* logits;
  uint16_t* w3;
  int S;
  int32_t *ids, *counts, *offsets, *route_src, *route_pos;
  float* wts;
  int32_t *counts_all, *offsets_all, *src_all, *pos_all;
  void* dscratch;
  int32_t *plan_up, *plan_down, *num_tiles;
  long max_up, max_down;
  PlanSpec up, down;
  uint16_t *h, *h_s, *dU, *du, *du_s;
  float *U, *dz, *dxp, *dx_s;
  int32_t *koff, *row_of, *tok_of;
  int Rp, Tp;
  uint16_t *dUt, *ht, *dut, *xgt, *dYt, *hst, *dust, *xt;
  // the fused front: the normed rows the layer runs on, the fp32 gradient
  // reaching them, each row's 1 / rms and the norm weight's partial sums
  uint16_t* x_norm;
  float *dxn, *r_norm, *dwn_part;
  // a latent layer: the experts' rows x_lat, the latent combine y_lat, the
  // gradients dy_lat and dx_lat [T][L] (bf16), dx_lat W_lin [T][d] (fp32)
  // and the transposes y_lat^T, dx_lat^T [L][Tp]
  uint16_t *x_lat, *y_lat, *dy_lat, *dx_lat, *y_latt, *dx_latt;
  float* dxl32;
  // split-K partials of the recomputed x_lat (as the forward's)
  int S_lin;
  float* part_lat;
};

size_t carve_backward(const moe_layer_desc* d, int T, void* ws, BwdBufs* b) {
  Carver c(ws);
  const int E = d->E, K = d->K, F = d->F, Fs = d->F_shared, D = d->d, L = d->d_latent;
  const int De = L ? L : D;  // the experts' input width
  const int Tc = T > 0 ? T : 1;
  const long R = (long)Tc * K;
  b->S = router_bf16_splits(Tc, D, E);
  b->w3 = c.take<uint16_t>((size_t)E * 3 * router_plane_width(D));
  b->logits = c.take<float>((size_t)b->S * Tc * E);
  b->ids = c.take<int32_t>(R);
  b->wts = c.take<float>(R);
  b->counts = c.take<int32_t>(E);
  b->offsets = c.take<int32_t>(E + 1);
  b->route_src = c.take<int32_t>(R);
  b->route_pos = c.take<int32_t>(R);
  if (d->capacity_factor > 0.0f) {
    b->counts_all = c.take<int32_t>(E);
    b->offsets_all = c.take<int32_t>(E + 1);
    b->src_all = c.take<int32_t>(R);
    b->pos_all = c.take<int32_t>(R);
  } else {
    b->counts_all = b->offsets_all = b->src_all = b->pos_all = nullptr;
  }
  b->dscratch = c.take<char>(dispatch_scratch_bytes(Tc, E));
  b->up = PlanSpec{E, Fs ? Tc : 0, ceil_div(F, kTileN), ceil_div(Fs > 0 ? Fs : 1, kTileN)};
  b->down = PlanSpec{E, Fs ? Tc : 0, ceil_div(De, kTileN), ceil_div(D, kTileN)};
  b->max_up = plan_max_tiles(b->up, R);
  b->max_down = plan_max_tiles(b->down, R);
  b->plan_up = c.take<int32_t>(2 * (size_t)b->max_up + 2);
  b->plan_down = c.take<int32_t>(2 * (size_t)b->max_down + 2);
  b->num_tiles = c.take<int32_t>(2);
  b->h = c.take<uint16_t>((size_t)R * F);
  b->h_s = Fs ? c.take<uint16_t>((size_t)Tc * Fs) : nullptr;
  b->U = c.take<float>((size_t)R * De);
  b->dz = c.take<float>(R);
  b->dU = c.take<uint16_t>((size_t)R * De);
  b->du = c.take<uint16_t>((size_t)R * F);
  b->du_s = Fs ? c.take<uint16_t>((size_t)Tc * Fs) : nullptr;
  b->dxp = c.take<float>((size_t)R * De);
  b->dx_s = Fs ? c.take<float>((size_t)Tc * D) : nullptr;
  // transposed operands of the weight gradients: each expert's rows padded
  // to a multiple of 8 columns (at most 7 E extra), group 0's T rows to Tp
  b->Rp = (int)((R + 7L * E + 7) / 8 * 8);
  b->Tp = (Tc + 7) / 8 * 8;
  b->koff = c.take<int32_t>(E + 1);
  b->row_of = c.take<int32_t>(b->Rp);
  b->tok_of = c.take<int32_t>(b->Rp);
  b->dUt = c.take<uint16_t>((size_t)De * b->Rp);
  b->ht = c.take<uint16_t>((size_t)F * b->Rp);
  b->dut = c.take<uint16_t>((size_t)F * b->Rp);
  b->xgt = c.take<uint16_t>((size_t)De * b->Rp);
  b->dYt = (Fs || L) ? c.take<uint16_t>((size_t)D * b->Tp) : nullptr;
  b->hst = Fs ? c.take<uint16_t>((size_t)Fs * b->Tp) : nullptr;
  b->dust = Fs ? c.take<uint16_t>((size_t)Fs * b->Tp) : nullptr;
  b->xt = (Fs || L) ? c.take<uint16_t>((size_t)D * b->Tp) : nullptr;
  if (L) {
    b->x_lat = c.take<uint16_t>((size_t)Tc * L);
    b->y_lat = c.take<uint16_t>((size_t)Tc * L);
    b->dy_lat = c.take<uint16_t>((size_t)Tc * L);
    b->dx_lat = c.take<uint16_t>((size_t)Tc * L);
    b->y_latt = c.take<uint16_t>((size_t)L * b->Tp);
    b->dx_latt = c.take<uint16_t>((size_t)L * b->Tp);
    b->dxl32 = c.take<float>((size_t)Tc * D);
    b->S_lin = latent_splits(Tc, L, D);
    b->part_lat = b->S_lin > 1 ? c.take<float>((size_t)b->S_lin * Tc * L) : nullptr;
  } else {
    b->x_lat = b->y_lat = b->dy_lat = b->dx_lat = b->y_latt = b->dx_latt = nullptr;
    b->dxl32 = nullptr;
    b->S_lin = 1;
    b->part_lat = nullptr;
  }
  if (d->flags & MOE_FLAG_PRENORM_RESIDUAL) {
    b->x_norm = c.take<uint16_t>((size_t)Tc * D);
    b->dxn = c.take<float>((size_t)Tc * D);
    b->r_norm = c.take<float>(Tc);
    b->dwn_part = c.take<float>((size_t)rmsnorm_dw_blocks(Tc) * D);
  } else {
    b->x_norm = nullptr;
    b->dxn = b->r_norm = b->dwn_part = nullptr;
  }
  return c.off + kAlign;
}

moe_status check_backward(const moe_layer_desc* d, int T) {
  const moe_status st = check_desc(d, T);
  if (st != MOE_OK) return st;
  if (d->act_dtype != MOE_BF16 || (d->flags & ~(MOE_FLAG_ZERO_SKIP_DOWN | MOE_FLAG_PRENORM_RESIDUAL)))
    return MOE_ERR_UNSUPPORTED;
  // the norm's backward keeps a row in registers, as its forward
  if ((d->flags & MOE_FLAG_PRENORM_RESIDUAL) && d->d > 8192) return MOE_ERR_UNSUPPORTED;
  // byte offsets of the backward GEMMs' operands stay in 32 bits
  const long R = (long)(T > 0 ? T : 1) * d->K;
  const long Rp = R + 7L * d->E + 8;
  const long wmax = std::max(std::max(d->d, d->F), d->d_latent);
  if (wmax * Rp * 2 >= (1L << 31) || R * wmax * 4 >= (1L << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}
}  // namespace

size_t moe_backward_workspace_size(const moe_layer_desc* desc, int T) {
  if (check_backward(desc, T) != MOE_OK) return 0;
  BwdBufs b;
  return carve_backward(desc, T, nullptr, &b);
}

namespace {
// One dense bf16 product of the backward, C [M][N] = A [M][Kd] . B on the
// grouped GEMM kernel's dense form (group 0 alone): B packed [N][Kd]
// (B_NK, the forward's packing) or [Kd][N] strips (B_KN, the neuron-major
// packing); C bf16 or fp32, with an fp32 addend and a residual source
// (EPI_ADD_F32).
moe_status dense_product(const void* A, long lda, int M, const void* B, int b_mode, int N, int Kd, void* C,
                         long ldc, int c_f32, int epi, const float* addend, long ld_add, const void* resid,
                         hipStream_t s) {
  GemmArgs g = {};
  g.M_s = M;
  g.A_s = A;
  g.lda_s = lda;
  g.B_s = B;
  g.ldb_s = b_mode == B_KN ? N : Kd;
  g.b_packed = 1;
  g.N_s = N;
  g.Kd_s = Kd;
  g.C_s = C;
  g.ldc_s = ldc;
  g.c_s_f32 = c_f32;
  g.addend = addend;
  g.ld_add = ld_add;
  g.resid = resid;
  g.ksplit = 1;
  return hip_status(launch_gemm(g, 1, b_mode, epi, 0, s));
}

// The forward relation the backward differentiates, into the backward's
// workspace: logits, ids, gates, the dispatch (and the dropless one the
// router gradient walks), h, h_s and the routed outputs U (fp32), and for
// a latent layer x_lat and the latent combine y_lat (bf16).  With y_s
// non-NULL the shared expert's output is computed too (fp32 [T][d]).
moe_status backward_forward(const moe_layer_desc& d, const moe_layer_weights* w, const uint16_t* X, int T,
                            BwdBufs& b, float* y_s, hipStream_t s) {
  const int E = d.E, K = d.K, F = d.F, Fs = d.F_shared, D = d.d, L = d.d_latent;
  const int De = L ? L : D;
  if (b.x_norm) {
    // the fused front: the layer runs on the normed rows of the hidden state X
    MOE_TRY(launch_rmsnorm(X, w->w_norm, d.norm_eps, T, D, 1, b.x_norm, s));
    X = b.x_norm;
  }
  // the experts' rows: x, or a latent layer's x W_lin^T (rounded to bf16)
  const uint16_t* Xe = X;
  if (L) {
    if (b.S_lin > 1) {
      // split over K into fp32 partials, summed in order and rounded once,
      // as the forward computes it
      GemmArgs li = {};
      li.M_s = T;
      li.A_s = X;
      li.lda_s = D;
      li.B_s = w->w_latent_in;
      li.ldb_s = D;
      li.b_packed = 1;
      li.N_s = L;
      li.Kd_s = D;
      li.split_main = 1;
      li.ksplit = b.S_lin;
      li.C_s = b.part_lat;
      li.ldc_s = L;
      li.c_s_f32 = 1;
      li.split_stride = (long)T * L;
      MOE_TRY(launch_gemm(li, 1, B_NK, EPI_STORE, 0, s));
      MOE_TRY(launch_reduce_splits(b.part_lat, b.S_lin, (long)T * L, T, L, nullptr, 0, nullptr, b.x_lat, 1, s));
    } else {
      MOE_TRY2(dense_product(X, D, T, w->w_latent_in, B_NK, L, D, b.x_lat, L, 0, EPI_STORE, nullptr, 0, nullptr,
                             s));
    }
    Xe = b.x_lat;
  }
  MOE_TRY(launch_split_router_weight(w->w_router, E, D, b.w3, s));
  MOE_TRY(launch_router_gemm_bf16x3(X, T, D, b.w3, E, b.logits, b.S, s));
  MOE_TRY(launch_route(b.logits, b.S, w->bias, T, E, K, d.n_group, d.topk_group, d.norm_topk_prob ? 1 : 0,
                       d.routed_scaling_factor, b.ids, b.wts, s));
  PlanOut P{b.plan_up, b.plan_down, b.num_tiles, b.up, b.down};
  if (b.counts_all) {
    const int C = (int)capacity_slots(T, K, E, d.capacity_factor);
    MOE_TRY(launch_dispatch(b.ids, T, K, E, b.counts_all, b.offsets_all, b.src_all, b.pos_all, b.dscratch, nullptr, s));
    MOE_TRY(launch_capacity(b.counts_all, b.offsets_all, b.src_all, b.wts, E, C, b.counts, b.offsets, b.route_src,
                            b.route_pos, s));
    MOE_TRY(launch_plan(b.offsets, &P, s));
  } else {
    MOE_TRY(launch_dispatch(b.ids, T, K, E, b.counts, b.offsets, b.route_src, b.route_pos, b.dscratch, &P, s));
  }
  GemmArgs up = {};
  up.E = E;
  up.offsets = b.offsets;
  up.gather = b.route_src;
  up.gdiv = K;
  up.A = Xe;
  up.lda = De;
  up.B = w->w_up;
  up.strideB = (long)F * De;
  up.ldb = De;
  up.b_packed = 1;
  up.N = F;
  up.Kd = De;
  up.C = b.h;
  up.ldc = F;
  up.M_s = Fs ? T : 0;
  up.A_s = X;
  up.lda_s = D;
  up.B_s = w->w_up_shared;
  up.ldb_s = D;
  up.N_s = Fs;
  up.Kd_s = D;
  up.C_s = b.h_s;
  up.ldc_s = Fs;
  up.plan = b.plan_up;
  up.num_tiles = b.num_tiles;
  up.ksplit = 1;
  MOE_TRY(launch_gemm(up, 1, B_NK, EPI_RELU2, (int)b.max_up, s));
  GemmArgs dn = {};
  dn.E = E;
  dn.offsets = b.offsets;
  dn.A = b.h;
  dn.lda = F;
  dn.B = w->w_down_t;
  dn.strideB = (long)F * De;
  dn.ldb = De;
  dn.b_packed = 1;
  dn.N = De;
  dn.Kd = F;
  dn.C = b.U;  // fp32: q = <dY, U> feeds a difference of gate terms
  dn.ldc = De;
  dn.c_f32 = 1;
  if (y_s && Fs) {
    dn.M_s = T;
    dn.A_s = b.h_s;
    dn.lda_s = Fs;
    dn.B_s = w->w_down_shared_t;
    dn.ldb_s = D;
    dn.N_s = D;
    dn.Kd_s = Fs;
    dn.C_s = y_s;
    dn.ldc_s = D;
    dn.c_s_f32 = 1;
  }
  dn.plan = b.plan_down;
  dn.num_tiles = b.num_tiles + 1;
  dn.ksplit = 1;
  MOE_TRY(launch_gemm(dn, 1, B_KN, EPI_STORE, (int)b.max_down, s));
  // the latent combine (routes in ascending id, fp32, one rounding)
  if (L) MOE_TRY(launch_combine_y32(b.U, b.wts, b.ids, b.route_pos, nullptr, T, K, L, nullptr, b.y_lat, s));
  return MOE_OK;
}

// Argument checks shared by the training forward and the backward.
moe_status check_backward_call(const moe_layer_desc* desc, const moe_layer_weights* w, int T) {
  moe_status st = check_backward(desc, T);
  if (st != MOE_OK) return st;
  if (!w) return MOE_ERR_INVALID_ARG;
  if (!w->w_router || !w->w_up || !w->w_down_t) return MOE_ERR_INVALID_ARG;
  if (desc->F_shared && (!w->w_up_shared || !w->w_down_shared_t)) return MOE_ERR_INVALID_ARG;
  if ((desc->flags & MOE_FLAG_PRENORM_RESIDUAL) && !w->w_norm) return MOE_ERR_INVALID_ARG;
  if (desc->d_latent && (!w->w_latent_in || !w->w_latent_out)) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {w->w_up, w->w_down_t, w->w_up_shared, w->w_down_shared_t, w->w_norm,
                        desc->d_latent ? w->w_latent_in : nullptr, desc->d_latent ? w->w_latent_out : nullptr};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}
}  // namespace

moe_status moe_layer_forward_train(const moe_layer_desc* desc, const moe_layer_weights* w, const void* x, int T,
                                   void* out, void* ws, size_t ws_bytes, moe_stream_t stream) {
  moe_status st = check_backward_call(desc, w, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(out)) return MOE_ERR_UNSUPPORTED;
  BwdBufs b;
  const size_t need = carve_backward(desc, T, nullptr, &b);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  carve_backward(desc, T, ws, &b);
  hipStream_t s = (hipStream_t)stream;
  const moe_layer_desc& d = *desc;
  // the shared expert's output goes to dx_s, a buffer the backward only
  // writes after it has read everything the forward left
  MOE_TRY2(backward_forward(d, w, (const uint16_t*)x, T, b, b.dx_s, s));
  // with the fused front the hidden state joins the sum last (out = Y + H)
  if (d.d_latent)
    // out = y_lat W_lout^T + y_s (+ H), one rounding
    return dense_product(b.y_lat, d.d_latent, T, w->w_latent_out, B_NK, d.d, d.d_latent, out, d.d, 0, EPI_ADD_F32,
                         d.F_shared ? b.dx_s : nullptr, d.d, b.x_norm ? x : nullptr, s);
  return hip_status(launch_combine_y32(b.U, b.wts, b.ids, b.route_pos, d.F_shared ? b.dx_s : nullptr, T, d.K, d.d,
                                       b.x_norm ? x : nullptr, out, s));
}

moe_status moe_layer_backward_timed(const moe_layer_desc* desc, const moe_layer_weights* w,
                                    const moe_layer_weights_bwd* wb, const void* x, const void* dy, int T,
                                    const moe_layer_grads* g, void* ws, size_t ws_bytes, moe_stream_t stream,
                                    void* const* events, int saved) {
  moe_status st = check_backward_call(desc, w, T);
  if (st != MOE_OK) return st;
  if (!wb || !g) return MOE_ERR_INVALID_ARG;
  const moe_layer_desc& d = *desc;
  const int E = d.E, K = d.K, F = d.F, Fs = d.F_shared, D = d.d, L = d.d_latent;
  const int De = L ? L : D;  // the experts' input width
  if (!wb->w_up_nm || !wb->w_down_nm) return MOE_ERR_INVALID_ARG;
  if (Fs && (!wb->w_up_shared_nm || !wb->w_down_shared_nm)) return MOE_ERR_INVALID_ARG;
  if (L && (!wb->w_latent_in_nm || !wb->w_latent_out_nm)) return MOE_ERR_INVALID_ARG;
  const bool prenorm = (d.flags & MOE_FLAG_PRENORM_RESIDUAL) != 0;
  if (!g->dw_router || !g->dw_up || !g->dw_down || (Fs && (!g->dw_up_shared || !g->dw_down_shared)) ||
      (prenorm && !g->dw_norm) || (L && (!g->dw_latent_in || !g->dw_latent_out)))
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !dy || !g->dx) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {x, dy, g->dx, g->dw_router, g->dw_up, g->dw_down, g->dw_up_shared, g->dw_down_shared,
                        wb->w_up_nm, wb->w_down_nm, wb->w_up_shared_nm, wb->w_down_shared_nm,
                        prenorm ? g->dw_norm : nullptr, L ? g->dw_latent_in : nullptr,
                        L ? g->dw_latent_out : nullptr, L ? wb->w_latent_in_nm : nullptr,
                        L ? wb->w_latent_out_nm : nullptr};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MOE_ERR_UNSUPPORTED;
  BwdBufs b;
  const size_t need = carve_backward(desc, T, nullptr, &b);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  carve_backward(desc, T, ws, &b);
  hipStream_t s = (hipStream_t)stream;
  // with the fused front, x is the hidden state H and the layer's steps run
  // on its normed rows (recomputed below, or left by the training forward)
  const uint16_t* H = (const uint16_t*)x;
  const uint16_t* X = prenorm ? b.x_norm : H;
  const uint16_t* DY = (const uint16_t*)dy;
  // a latent layer's experts see x_lat and the combine's gradient dy_lat
  const uint16_t* Xe = L ? b.x_lat : X;
  const uint16_t* DYe = L ? b.dy_lat : DY;
  const long R = (long)T * K;
  auto rec = [&](int i) -> hipError_t {
    return events ? hipEventRecord((hipEvent_t)events[i], s) : hipSuccess;
  };
  // every selected route's logit gradient reaches the router weight, also a
  // dropped route's: the router gradient walks the dropless dispatch
  const int32_t* r_off = b.counts_all ? b.offsets_all : b.offsets;
  const int32_t* r_src = b.counts_all ? b.src_all : b.route_src;

  // ---- the forward relation: recomputed with the forward's kernels, or
  // left in the workspace by moe_layer_forward_train ----
  MOE_TRY(rec(2 * MOE_BWD_STAGE_FORWARD));
  if (!saved) MOE_TRY2(backward_forward(d, w, H, T, b, nullptr, s));
  MOE_TRY(rec(2 * MOE_BWD_STAGE_FORWARD + 1));

  // ---- combine and gate adjoints, router projection ----
  MOE_TRY(rec(2 * MOE_BWD_STAGE_GATES));
  // a latent layer: dy_lat = dY W_lout (W_lout [d][L] read as [K][N] strips)
  if (L)
    MOE_TRY2(dense_product(DY, D, T, wb->w_latent_out_nm, B_KN, L, D, b.dy_lat, L, 0, EPI_STORE, nullptr, 0,
                           nullptr, s));
  MOE_TRY(launch_gate_grad(DYe, b.U, b.logits, b.S, (long)T * E, b.ids, b.wts, b.route_pos, T, E, K, De,
                           d.norm_topk_prob ? 1 : 0, d.routed_scaling_factor, b.dz, b.dU, s));
  MOE_TRY(launch_router_grad(X, D, K, E, r_off, r_src, b.dz, g->dw_router, s));
  MOE_TRY(rec(2 * MOE_BWD_STAGE_GATES + 1));
  MOE_TRY(rec(2 * MOE_BWD_STAGE_DH));

  // ---- input-side products: dh -> du (ReLU^2'), du -> dx rows ----
  GemmArgs gh = {};
  gh.E = E;
  gh.offsets = b.offsets;
  gh.A = b.dU;
  gh.lda = De;
  gh.B = wb->w_down_nm;
  gh.strideB = (long)De * F;
  gh.ldb = F;
  gh.b_packed = 1;
  gh.N = F;
  gh.Kd = De;
  gh.C = b.du;
  gh.ldc = F;
  gh.aux = b.h;
  gh.M_s = Fs ? T : 0;
  gh.A_s = DY;
  gh.lda_s = D;
  gh.B_s = wb->w_down_shared_nm;
  gh.ldb_s = Fs;
  gh.N_s = Fs;
  gh.Kd_s = D;
  gh.C_s = b.du_s;
  gh.ldc_s = Fs;
  gh.aux_s = b.h_s;
  gh.plan = b.plan_up;
  gh.num_tiles = b.num_tiles;
  gh.ksplit = 1;
  MOE_TRY(launch_gemm(gh, 1, B_KN, EPI_DRELU2, (int)b.max_up, s));
  MOE_TRY(rec(2 * MOE_BWD_STAGE_DH + 1));
  MOE_TRY(rec(2 * MOE_BWD_STAGE_DX));
  GemmArgs gx = {};
  gx.E = E;
  gx.offsets = b.offsets;
  gx.A = b.du;
  gx.lda = F;
  gx.B = wb->w_up_nm;
  gx.strideB = (long)F * De;
  gx.ldb = De;
  gx.b_packed = 1;
  gx.N = De;
  gx.Kd = F;
  gx.C = b.dxp;
  gx.ldc = De;
  gx.c_f32 = 1;
  gx.M_s = Fs ? T : 0;
  gx.A_s = b.du_s;
  gx.lda_s = Fs;
  gx.B_s = wb->w_up_shared_nm;
  gx.ldb_s = D;
  gx.N_s = D;
  gx.Kd_s = Fs;
  gx.C_s = b.dx_s;
  gx.ldc_s = D;
  gx.c_s_f32 = 1;
  gx.plan = b.plan_down;
  gx.num_tiles = b.num_tiles + 1;
  gx.ksplit = 1;
  MOE_TRY(launch_gemm(gx, 1, B_KN, EPI_STORE, (int)b.max_down, s));
  // the routes' input gradients: gathered per token into dx (or, for a
  // latent layer, into dx_lat, then carried back by dx_lat W_lin)
  const float* dxp_full = b.dxp;
  if (L) {
    MOE_TRY(launch_dx_combine(b.dxp, nullptr, nullptr, nullptr, b.ids, b.route_pos, b.dz, T, K, L, b.dx_lat,
                              nullptr, s));
    MOE_TRY2(dense_product(b.dx_lat, L, T, wb->w_latent_in_nm, B_KN, D, L, b.dxl32, D, 1, EPI_STORE, nullptr, 0,
                           nullptr, s));
    dxp_full = nullptr;
  }
  if (prenorm) {
    // the gradient reaching the normed rows (fp32), then through the norm:
    // dH = dY + RMSNorm'(H)^T dx (the residual's path) and dw_norm
    MOE_TRY(launch_dx_combine(dxp_full, b.dx_s, b.dxl32, w->w_router, b.ids, b.route_pos, b.dz, T, K, D, nullptr,
                              b.dxn, s));
    MOE_TRY(launch_rmsnorm_bwd(H, (const uint16_t*)w->w_norm, d.norm_eps, T, D, b.dxn, DY, (uint16_t*)g->dx,
                               g->dw_norm, b.r_norm, b.dwn_part, s));
  } else {
    MOE_TRY(launch_dx_combine(dxp_full, b.dx_s, b.dxl32, w->w_router, b.ids, b.route_pos, b.dz, T, K, D,
                              (uint16_t*)g->dx, nullptr, s));
  }
  MOE_TRY(rec(2 * MOE_BWD_STAGE_DX + 1));

  // ---- weight gradients: per expert, products over its rows ----
  MOE_TRY(rec(2 * MOE_BWD_STAGE_TRANSPOSE));
  MOE_TRY(launch_wgrad_map(b.offsets, b.route_src, E, K, b.Rp, b.koff, b.row_of, b.tok_of, s));
  MOE_TRY(launch_transpose_rows(b.dU, De, De, b.row_of, 0, b.Rp, b.dUt, b.Rp, s));
  MOE_TRY(launch_transpose_rows(b.h, F, F, b.row_of, 0, b.Rp, b.ht, b.Rp, s));
  MOE_TRY(launch_transpose_rows(b.du, F, F, b.row_of, 0, b.Rp, b.dut, b.Rp, s));
  MOE_TRY(launch_transpose_rows(Xe, De, De, b.tok_of, 0, b.Rp, b.xgt, b.Rp, s));
  if (Fs || L) {
    MOE_TRY(launch_transpose_rows(DY, D, D, nullptr, T, b.Tp, b.dYt, b.Tp, s));
    MOE_TRY(launch_transpose_rows(X, D, D, nullptr, T, b.Tp, b.xt, b.Tp, s));
  }
  if (Fs) {
    MOE_TRY(launch_transpose_rows(b.h_s, Fs, Fs, nullptr, T, b.Tp, b.hst, b.Tp, s));
    MOE_TRY(launch_transpose_rows(b.du_s, Fs, Fs, nullptr, T, b.Tp, b.dust, b.Tp, s));
  }
  if (L) {
    MOE_TRY(launch_transpose_rows(b.y_lat, L, L, nullptr, T, b.Tp, b.y_latt, b.Tp, s));
    MOE_TRY(launch_transpose_rows(b.dx_lat, L, L, nullptr, T, b.Tp, b.dx_latt, b.Tp, s));
  }
  MOE_TRY(rec(2 * MOE_BWD_STAGE_TRANSPOSE + 1));
  MOE_TRY(rec(2 * MOE_BWD_STAGE_DW_DOWN));
  // dW_down[e] [d][F] = dU^T h over the expert's rows
  GemmArgs wd = {};
  wd.wgrad = 1;
  wd.E = E;
  wd.koff = b.koff;
  wd.M = De;
  wd.A = b.dUt;
  wd.lda = b.Rp;
  wd.B = b.ht;
  wd.ldb = b.Rp;
  wd.N = F;
  wd.C = g->dw_down;
  wd.c_f32 = 1;
  wd.M_s = D;
  wd.A_s = b.dYt;
  wd.lda_s = b.Tp;
  wd.B_s = b.hst;
  wd.ldb_s = b.Tp;
  wd.N_s = Fs;
  wd.Kd_s = Fs ? b.Tp : 0;
  wd.C_s = g->dw_down_shared;
  wd.ldc_s = Fs;
  wd.c_s_f32 = 1;
  wd.ksplit = 1;
  MOE_TRY(launch_gemm(wd, 1, B_NKP, EPI_STORE, 0, s));
  if (L) {
    // dW_lout [d][L] = dY^T y_lat
    GemmArgs wl = {};
    wl.wgrad = 1;
    wl.M_s = D;
    wl.A_s = b.dYt;
    wl.lda_s = b.Tp;
    wl.B_s = b.y_latt;
    wl.ldb_s = b.Tp;
    wl.N_s = L;
    wl.Kd_s = b.Tp;
    wl.C_s = g->dw_latent_out;
    wl.ldc_s = L;
    wl.c_s_f32 = 1;
    wl.ksplit = 1;
    MOE_TRY(launch_gemm(wl, 1, B_NKP, EPI_STORE, 0, s));
  }
  MOE_TRY(rec(2 * MOE_BWD_STAGE_DW_DOWN + 1));
  MOE_TRY(rec(2 * MOE_BWD_STAGE_DW_UP));
  // dW_up[e] [F][d] = du^T x over the expert's rows
  GemmArgs wu = {};
  wu.wgrad = 1;
  wu.E = E;
  wu.koff = b.koff;
  wu.M = F;
  wu.A = b.dut;
  wu.lda = b.Rp;
  wu.B = b.xgt;
  wu.ldb = b.Rp;
  wu.N = De;
  wu.C = g->dw_up;
  wu.c_f32 = 1;
  wu.M_s = Fs;
  wu.A_s = b.dust;
  wu.lda_s = b.Tp;
  wu.B_s = b.xt;
  wu.ldb_s = b.Tp;
  wu.N_s = D;
  wu.Kd_s = Fs ? b.Tp : 0;
  wu.C_s = g->dw_up_shared;
  wu.ldc_s = D;
  wu.c_s_f32 = 1;
  wu.ksplit = 1;
  MOE_TRY(launch_gemm(wu, 1, B_NKP, EPI_STORE, 0, s));
  if (L) {
    // dW_lin [L][d] = dx_lat^T x
    GemmArgs wi = {};
    wi.wgrad = 1;
    wi.M_s = L;
    wi.A_s = b.dx_latt;
    wi.lda_s = b.Tp;
    wi.B_s = b.xt;
    wi.ldb_s = b.Tp;
    wi.N_s = D;
    wi.Kd_s = b.Tp;
    wi.C_s = g->dw_latent_in;
    wi.ldc_s = D;
    wi.c_s_f32 = 1;
    wi.ksplit = 1;
    MOE_TRY(launch_gemm(wi, 1, B_NKP, EPI_STORE, 0, s));
  }
  MOE_TRY(rec(2 * MOE_BWD_STAGE_DW_UP + 1));
  (void)R;
  return MOE_OK;
}

moe_status moe_layer_backward(const moe_layer_desc* desc, const moe_layer_weights* w,
                              const moe_layer_weights_bwd* wb, const void* x, const void* dy, int T,
                              const moe_layer_grads* g, void* ws, size_t ws_bytes, moe_stream_t stream) {
  return moe_layer_backward_timed(desc, w, wb, x, dy, T, g, ws, ws_bytes, stream, nullptr, 0);
}

moe_status moe_layer_backward_saved(const moe_layer_desc* desc, const moe_layer_weights* w,
                                    const moe_layer_weights_bwd* wb, const void* x, const void* dy, int T,
                                    const moe_layer_grads* g, void* ws, size_t ws_bytes, moe_stream_t stream) {
  return moe_layer_backward_timed(desc, w, wb, x, dy, T, g, ws, ws_bytes, stream, nullptr, 1);
}

moe_status moe_layer_forward(const moe_layer_desc* desc, const moe_layer_weights* w, const void* x,
                             int T, void* out, void* ws, size_t ws_bytes, moe_stream_t stream) {
  return moe_layer_forward_timed(desc, w, x, T, out, ws, ws_bytes, stream, nullptr);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// moe_layer_forward_noalloc: moe_layer_forward with its workspace in a
// static device array instead of a caller's buffer, for callers that cannot
// allocate.  Each GPU the library runs on holds its own copy of `scratch`
// from the module's load until the process ends.  Host code never passes
// `scratch` itself to a kernel (on the host it names a stand-in, not the
// device copy): the device address of each GPU's copy is looked up once,
// with that GPU current, and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of the current GPU's `scratch`.
moe_status scratch_address(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return MOE_OK;
}
}  // namespace

extern "C" moe_status moe_layer_forward_noalloc(const moe_layer_desc* desc, const moe_layer_weights* w,
                                                const void* x, int T, void* out, moe_stream_t stream) {
  const moe_status st = check_desc(desc, T);
  if (st != MOE_OK) return st;
  FwdBufs b;
  if (carve_forward(desc, T, nullptr, &b) > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_UNSUPPORTED;
  void* ws = nullptr;
  const moe_status sa = scratch_address(&ws);
  if (sa != MOE_OK) return sa;
  // the forward path reads nothing of its workspace before writing it, so
  // what an earlier call left in `scratch` needs no clearing
  return moe_layer_forward_timed(desc, w, x, T, out, ws, MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}
