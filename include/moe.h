/*
 * moe.h -- C ABI of libmoe, the forward pass of a routed ReLU^2
 * mixture-of-experts layer (Nemotron-style) on AMD Instinct MI355X (gfx950).
 *
 * The layer: an fp32 sigmoid router with bias-corrected, group-limited
 * top-k selection; dispatch of the (token, slot) routes into expert-major
 * rows; routed experts W_down relu(W_up x)^2 with no gate; an always-active
 * shared ReLU^2 expert; and a weighted combine back to token rows.
 *
 * Sources, by page and section:
 *  [circuit]   "Nemotron is not one circuit: Mamba, attention and MoE
 *              routing" (shivasnotes.com): "The Four Layer Kinds CKE Must
 *              Preserve", "The Router Is A Deterministic Algorithm", "The C
 *              Kernel Contract", "Routing Is Cheap; Expert Memory Is The
 *              Hard Part".
 *  [M6.1]      "M6.1 - Routed Capacity: MoE Experts, Routers, and Token
 *              Dispatch" (transformer-system.numinens.com): 0x04A, 0x05A,
 *              0x05B, 0x05E, 0x05F.
 *  [NemotronH] "NemotronH (Nemotron 3.5 Lightning, Bolt, Super VL)"
 *              (tandemllm docs v0.13.0): "Arithmetic".
 *  [8GB]       hot.atechcom.net write-up of Nemotron-3.5-Super on an 8 GB
 *              card: "The only number that matters: bytes per token",
 *              "The engine, step by step" (item 4, skipping zeros).
 *
 * Conventions common to every entry point
 *  - Every pointer argument is DEVICE memory owned by the caller, unless the
 *    argument says otherwise.  The library never allocates or frees device
 *    memory and keeps no state between calls; scratch space comes only from
 *    the caller's workspace (ws, ws_bytes).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream).  No call synchronises the host.  Two calls that share a
 *    workspace or an output must be ordered by the caller (same stream).
 *  - Every call validates its arguments on the host before any launch; on
 *    any error it launches nothing and returns the status.  T == 0 (no rows)
 *    is a successful no-op once the sizes and the layer description are
 *    valid: it reads no row pointer (x, out, ids, logits, ... may be NULL,
 *    as an empty tensor's are) and writes nothing.
 *  - Activations are row-major.  The expert, shared-expert and latent
 *    weight matrices are passed in the packed layout that moe_pack_weight
 *    writes, from PyTorch nn.Linear storage [out, in] ([M6.1] 0x04A) for the
 *    up and latent projections and from neuron-major storage for the down
 *    projections (the transpose of the PyTorch [d_e, F] storage: row f holds
 *    the d_e outputs of hidden neuron f, so skipping a zero neuron skips one
 *    row).  Shapes below name the logical matrix.  The router weight is
 *    plain row-major [E, d].
 *  - bf16 is IEEE-754 binary32 truncated to its upper 16 bits (bfloat16);
 *    bf16 tensors are passed as 2-byte elements.
 *  - Result dtypes: ids/offsets/maps int32; router logits and gate weights
 *    fp32; expert outputs and the layer output in the activation dtype.
 *  - Determinism: no floating-point atomics are used; repeated calls with
 *    the same inputs give bitwise-identical outputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *moe_stream_t; /* a hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* an argument breaks the method's constraints  */
  MOE_ERR_UNSUPPORTED = 2, /* valid for the method, not for this library    */
  MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required    */
  MOE_ERR_HIP = 4          /* the HIP runtime reported a launch error       */
} moe_status;

/* MOE_FP8_E4M3: the OCP 8-bit float E4M3 ("FN": 4 exponent bits with bias
 * 7, 3 mantissa bits, subnormals, no infinities, S.1111.111 the only NaN,
 * 448 the largest finite value), one byte per element.  A storage type for
 * expert weights only (moe_quantize_fp8, moe_pack_weight,
 * MOE_FLAG_FP8_EXPERTS, moe_experts_fp8), never an activation dtype. */
/* MOE_MXFP4: MXFP4 of the OCP Microscaling Formats specification (v1.0):
 * 4-bit E2M1 elements (sign, 2 exponent bits with bias 1, 1 mantissa bit;
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte (element 2i in the
 * low nibble), and one E8M0 scale byte 2^(e - 127) per block of 32
 * consecutive elements along a matrix's input dimension.  A storage type
 * for expert weights only (moe_quantize_mxfp4, moe_pack_weight,
 * MOE_FLAG_MXFP4_EXPERTS, moe_experts_mxfp4). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2, MOE_MXFP4 = 3 } moe_dtype;

enum {
  /* Decode path: the down projections read only the rows of the
   * neuron-major down weights whose hidden neuron is non-zero after ReLU^2
   * for at least one row of the expert's batch (post-ReLU^2 zeros, [8GB]
   * "The engine, step by step", item 4).  Taken for bf16 batches of at most
   * 256 rows (and at most 8192 routes, widths at most 4096); for other
   * calls the flag is a hint and the grouped GEMMs run.  The result is the
   * same layer either way (the decode path keeps each route's down output
   * in fp32 until the combine). */
  MOE_FLAG_ZERO_SKIP_DOWN = 1,
  /* The layer output is added to `out` (out = out + Y) inside the final
   * fp32 sum instead of overwriting it: the residual add that follows the
   * layer ([M6.1] 0x05F keeps the residual outside Y itself). */
  MOE_FLAG_ACCUMULATE_OUT = 2,
  /* Fused front and back of the layer (moe_layer_forward only): x is the
   * hidden state H; the layer runs on RMSNorm(H) * w_norm (moe_rmsnorm,
   * with desc.norm_eps) and H joins the final fp32 sum last, so out =
   * round(Y + H): [circuit] "The Four Layer Kinds CKE Must Preserve"
   * (RMSNorm -> router -> ... -> residual), [M6.1] 0x06F.1 (R = H + Y).
   * Not combinable with MOE_FLAG_ACCUMULATE_OUT. */
  MOE_FLAG_PRENORM_RESIDUAL = 4,
  /* FP8 experts, weights only (W8A16): the routed and shared expert
   * matrices (w_up, w_down_t, w_up_shared, w_down_shared_t) are E4M3 codes
   * written by moe_quantize_fp8 (one fp32 scale per output channel: per
   * hidden neuron for the up projections, per output column for the down
   * projections) and packed by moe_pack_weight with dt MOE_FP8_E4M3; the
   * scales are passed in the w_*_scale fields.  A weight's value is scale *
   * E4M3 value, exact; activations, the hidden h and the latent projections
   * stay bf16 and every product is accumulated in fp32, so the layer is the
   * bf16 layer on the dequantised weights.  [circuit] "What CKE Has
   * Actually Established" (quantised expert forward variants) and "Why This
   * Architecture Is Especially Interesting On CPUs" (quantised expert
   * weights and the compute-to-bandwidth balance); [NemotronH] and [8GB]
   * serve the experts from FP8 / 4-bit checkpoints.  Needs act_dtype
   * MOE_BF16 and d, F, F_shared, d_latent multiples of 16. */
  MOE_FLAG_FP8_EXPERTS = 8,
  /* MXFP4 experts, weights only (W4A16): every routed and shared expert
   * matrix is quantised by moe_quantize_mxfp4 (E2M1 codes with an E8M0
   * scale per 32 inputs: blocks along the model width for the up
   * projections, along the hidden neurons for the down projections) and
   * its codes packed by moe_pack_weight with dt MOE_MXFP4.  The down
   * projections are passed twice, as the same codes in two packings:
   * w_down_t (NEURON_MAJOR, read by the decode path) and w_down /
   * w_down_shared ([OUT_IN], read by the grouped GEMMs); the scales go in
   * the w_*_e8 fields.  A weight's value is 2^(e - 127) * E2M1 value,
   * widened exactly to bf16; activations, h and the latent projections stay
   * bf16 and every product is accumulated in fp32, so the layer is the bf16
   * layer on the dequantised weights.  [8GB] "The only number that
   * matters: bytes per token" (4-bit experts with block scales).  Needs
   * act_dtype MOE_BF16, d, F, F_shared, d_latent multiples of 32; not
   * combinable with MOE_FLAG_FP8_EXPERTS. */
  MOE_FLAG_MXFP4_EXPERTS = 16,
  /* W4A8 experts (with MOE_FLAG_MXFP4_EXPERTS only): the inputs of both
   * expert products -- the rows an up projection reads (x, or the latent
   * rows) and the ReLU^2 output a down projection reads -- are MXFP8 (OCP
   * Microscaling Formats v1.0: E4M3 elements, one E8M0 scale per 32 values
   * along the product's reduction axis, shared exponent floor(log2 amax) -
   * 8, round to nearest even, saturation at 448; moe_quantize_mxfp8's
   * rule), and the products run on the block-scaled MFMA with the MXFP4
   * weights, fp32 accumulation.  The ReLU^2 output is squared in fp32 and
   * quantised from fp32; the down products' outputs, the combine and the
   * latent projections are as without the flag.  [8GB] "The only number
   * that matters: bytes per token" and [NemotronH] "How the engine runs
   * it" (experts from 4-bit block-scaled checkpoints).  Such calls run the
   * grouped GEMMs (MOE_FLAG_ZERO_SKIP_DOWN is a hint they do not take). */
  MOE_FLAG_MXFP8_ACTIVATIONS = 32
};

/* Limits of this library (MOE_ERR_UNSUPPORTED beyond them). */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 32
#define MOE_MAX_GROUPS 64

/* Layer description.  d: model width; E: routed experts; K: experts per
 * token; F: routed hidden width; F_shared: shared-expert hidden width (0 =
 * no shared expert); d_latent: width the routed experts run in (0 = they run
 * on d; otherwise a latent layer: x is projected to d_latent before the
 * experts and the combined result is projected back to d).
 * n_group/topk_group: group-limited selection (n_group = 1: none);
 * norm_topk_prob: normalise the selected weights to sum 1 before scaling;
 * routed_scaling_factor: multiplies the selected weights.
 * act_dtype: dtype of x, out and every expert/shared/latent weight; the
 * router weight and bias are fp32 whatever act_dtype is.
 * norm_eps: the RMSNorm epsilon (>= 0), read only with
 * MOE_FLAG_PRENORM_RESIDUAL.
 * capacity_factor: 0 = dropless; > 0 = the capacity-bounded variant: each
 * expert takes at most C = moe_capacity_slots(T, K, E, capacity_factor)
 * routes of the call, chosen by moe_dispatch_capacity's rule, and an
 * overflowed route contributes nothing (the token's other gates are not
 * renormalised).  Such calls run the grouped GEMMs (never the decode
 * path). */
typedef struct {
  int d, E, K, F, F_shared, d_latent;
  int n_group, topk_group, norm_topk_prob;
  float routed_scaling_factor;
  moe_dtype act_dtype;
  int flags; /* MOE_FLAG_* */
  float norm_eps;
  float capacity_factor;
} moe_layer_desc;

/* Weights (device pointers, act_dtype unless noted), d_e = d_latent ? d_latent : d.
 * Every matrix but the router's is packed by moe_pack_weight (kind in []). */
typedef struct {
  const float *w_router;        /* [E, d] fp32, plain row-major                 */
  const float *bias;            /* [E] fp32 selection-only correction, or NULL  */
  const void *w_up;             /* [E, F, d_e]  [OUT_IN]                        */
  const void *w_down_t;         /* [E, F, d_e]  [NEURON_MAJOR] down projections */
  const void *w_up_shared;      /* [F_shared, d] [OUT_IN], NULL when F_shared 0 */
  const void *w_down_shared_t;  /* [F_shared, d] [NEURON_MAJOR]                 */
  const void *w_latent_in;      /* [d_latent, d] [OUT_IN], NULL when d_latent 0 */
  const void *w_latent_out;     /* [d, d_latent] [OUT_IN]                       */
  const void *w_norm;           /* [d] RMSNorm weight, plain; read only with
                                   MOE_FLAG_PRENORM_RESIDUAL                    */
  /* per-output-channel fp32 scales, read only with MOE_FLAG_FP8_EXPERTS      */
  const float *w_up_scale;          /* [E, F]     one per hidden neuron        */
  const float *w_down_scale;        /* [E, d_e]   one per output column        */
  const float *w_up_shared_scale;   /* [F_shared] (NULL when F_shared is 0)    */
  const float *w_down_shared_scale; /* [d]        (NULL when F_shared is 0)    */
  /* read only with MOE_FLAG_MXFP4_EXPERTS: the down codes packed [OUT_IN]
   * for the grouped GEMMs, and the E8M0 scales, stored block-major (the
   * scale of output row o, input block j at [j][o])                        */
  const void *w_down;               /* [E, d_e, F]  [OUT_IN]                  */
  const void *w_down_shared;        /* [d, F_shared] [OUT_IN]                 */
  const uint8_t *w_up_e8;           /* [E, d_e / 32, F]                       */
  const uint8_t *w_down_e8;         /* [E, F / 32, d_e]                       */
  const uint8_t *w_up_shared_e8;    /* [d / 32, F_shared]                     */
  const uint8_t *w_down_shared_e8;  /* [F_shared / 32, d]                     */
} moe_layer_weights;

/* ------------------------------------------------------------------------
 * FP8 quantisation of weights, done once when they are loaded: per row of
 * `rows` rows of C columns (plain row-major, the [out, in] storage, so one
 * scale per output channel), scale = amax / 448 in fp32 (1 for an all-zero
 * row) and code = E4M3(w / scale), the division in fp32 (correctly
 * rounded) and the encoding round-to-nearest-even, magnitudes past 448
 * saturating to 448 (so no NaN code is written; -0 keeps its sign).  Each
 * row's largest magnitude lands on 448.  [circuit] "What CKE Has Actually
 * Established" (quantised expert variants).
 *   w       [rows, C] in dt (MOE_BF16 or MOE_F32)
 *   codes   [rows, C] uint8 E4M3 (written);  scales [rows] fp32 (written)
 * The down projections are quantised from their [d_e, F] storage (one scale
 * per output column) and transposed to neuron-major before packing.
 * Errors: INVALID_ARG for rows < 0, C < 1, an unknown dtype, NULL pointers
 *   (rows > 0).  rows == 0 is a no-op. */
moe_status moe_quantize_fp8(const void *w, moe_dtype dt, long rows, int C, uint8_t *codes,
                            float *scales, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * MXFP4 quantisation of weights (OCP Microscaling Formats v1.0), done once
 * when they are loaded: G matrices of R rows and C columns in [out, in]
 * storage, blocks of 32 consecutive columns.  Per block: amax in fp32,
 * shared = floor(log2 amax) - 2 clamped to [-127, 127] (-127 for an
 * all-zero block), scale byte = shared + 127, and each element's code =
 * E2M1(w / 2^shared) rounded to nearest, ties to the even code, magnitudes
 * past 6 saturating to 6 (-0 keeps its sign).  [8GB] "The only number
 * that matters: bytes per token".
 *   w       [G, R, C] in dt (MOE_BF16 or MOE_F32), plain row-major
 *   codes   [G, R, C / 2] bytes, element 2i of a row in the low nibble
 *   scales  [G, C / 32, R] bytes: block j of row r at scales[g][j][r]
 * Errors: INVALID_ARG for G, R < 0, C < 1, an unknown dtype, NULL pointers
 *   (G*R > 0); UNSUPPORTED for C % 32 != 0 or a matrix over 2^31 elements.
 *   G*R == 0 is a no-op. */
moe_status moe_quantize_mxfp4(const void *w, moe_dtype dt, int G, int R, int C, uint8_t *codes,
                              uint8_t *scales, moe_stream_t stream);

/* MXFP8 quantisation of activations (OCP Microscaling Formats v1.0), the
 * rule MOE_FLAG_MXFP8_ACTIVATIONS applies to the experts' inputs: rows of C
 * values, blocks of 32 consecutive values.  Per block: amax, shared =
 * floor(log2 amax) - 8 clamped to [-127, 127] (-127 for an all-zero
 * block), scale byte = shared + 127, and each value's E4M3 code of
 * v / 2^shared, nearest with ties to the even code, magnitudes at or past
 * 448 saturating to 448 (no NaN code is written; -0 keeps its sign).
 *   x       [rows, C] bf16 (dt MOE_BF16)
 *   codes   [rows, C] uint8 E4M3 (written)
 *   scales  [C / 32, ld] uint8, block-major: block j of row r at
 *           scales[j * ld + r] (written; ld >= rows)
 * Errors: INVALID_ARG for rows < 0, C < 1, ld < rows, a dtype other than
 *   MOE_BF16, NULL pointers (rows > 0); UNSUPPORTED for C % 32 != 0 or
 *   unaligned x / codes (16 bytes).  rows == 0 is a no-op. */
moe_status moe_quantize_mxfp8(const void *x, moe_dtype dt, int rows, int C, uint8_t *codes, uint8_t *scales,
                              long ld, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Weight packing, done once when the weights are loaded.  G matrices of R
 * rows and C columns, plain row-major in src ([G, R, C]), are written to dst
 * (same size, G consecutive packed matrices) rearranged for the kernels'
 * tiles: a performance layout, not a step of the method.
 *   MOE_PACK_OUT_IN (up, shared up, latent in/out; R = out, C = in): rows in
 *     tiles of 256 (the last tile rn = R - r0 rows), each tile stored as its
 *     column steps of 32 (the last step kw = C - c0 columns), each step a
 *     row-major [rn, kw] block.  Element (r, c) of a matrix sits at
 *     r0*C + c0*rn + (r - r0)*kw + (c - c0), r0 = r & ~255, c0 = c & ~31.
 *   MOE_PACK_NEURON_MAJOR (routed and shared down_t; R = hidden neurons,
 *     C = outputs): columns in strips of 256 (the last strip cn = C - c0
 *     columns), each strip row-major [R, cn].  Element (r, c) sits at
 *     c0*R + r*cn + (c - c0), c0 = c & ~255.
 *   src, dst  device memory, distinct and not overlapping; dt sets the
 *             element size (MXFP4 codes half a byte, two per byte in
 *             element order; fp8 1 byte, bf16 2 bytes, fp32 4 bytes).
 * Errors: INVALID_ARG for G, R or C < 0, an unknown kind or dtype, NULL or
 *   overlapping src/dst (when G*R*C > 0); UNSUPPORTED for C % 8 != 0
 *   (C % 16 != 0 for MOE_FP8_E4M3, C % 32 for MOE_MXFP4), a matrix over
 *   2 GiB, or pointers not
 *   16-byte aligned.  G*R*C == 0 is a
 *   no-op. */
typedef enum { MOE_PACK_OUT_IN = 0, MOE_PACK_NEURON_MAJOR = 1 } moe_pack_kind;
moe_status moe_pack_weight(const void *src, moe_dtype dt, int G, int R, int C, int kind,
                           void *dst, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * RMSNorm: out[t] = round(x[t] / sqrt(mean_j x[t,j]^2 + eps) * w_norm) in
 * fp32 with one rounding to dt ([NemotronH] "Arithmetic": the RMS norm in
 * fp32 times the plain weight).  The fp32 sum of squares has a fixed order:
 * the row is cut into 8-element chunks, chunk c is added (square by square,
 * in element order) to partial sum c mod 64, and the 64 partials are added
 * in halving folds (j + j+32, then j + j+16, ...); every product and sum is
 * rounded to fp32 on its own; sqrt and the division are correctly rounded.
 * The result is therefore the same bits on every run and device.
 *   x, out [T, d] in dt (out may not overlap x);  w_norm [d] in dt
 * Errors: INVALID_ARG for T < 0, d < 1, eps < 0 or not finite, NULL
 *   pointers (T > 0); UNSUPPORTED for d % 8 != 0, d > 8192 or pointers not
 *   16-byte aligned. */
moe_status moe_rmsnorm(const void *x, const void *w_norm, float eps, int T, int d, moe_dtype dt,
                       void *out, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Router logits: logits[t, e] = sum_j x[t, j] * w_router[e, j], in fp32.
 * [M6.1] 0x04A (the router is nn.Linear(d, E) stored [E, d], Z = H W^T);
 * [NemotronH] "Arithmetic" (fp32 logits).
 *   x        [T, d] in `dt` (bf16 values are widened exactly)
 *   w_router [E, d] fp32
 *   logits   [T, E] fp32 (written)
 *   ws       scratch of at least moe_router_logits_workspace_size(T, d, E, dt)
 *            bytes (may be NULL when that size is 0)
 * Errors: INVALID_ARG for NULL pointers or sizes < 0 / E < 1;
 *         UNSUPPORTED for E > MOE_MAX_EXPERTS or d % 8 != 0;
 *         WORKSPACE when ws_bytes is too small. */
size_t moe_router_logits_workspace_size(int T, int d, int E, moe_dtype dt);
moe_status moe_router_logits(const void *x, moe_dtype dt, int T, int d,
                             const float *w_router, int E, float *logits,
                             void *ws, size_t ws_bytes, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Group-limited sigmoid router, one row per token.  [circuit] "The Router Is
 * A Deterministic Algorithm" and "The C Kernel Contract" (scores [R][E],
 * optional correction_bias [E], indices [R][K], weights [R][K], n_group,
 * topk_group, norm_topk_prob, routed_scaling_factor); [NemotronH]
 * "Arithmetic" (sigmoid, bias for the choice only, ties to the lower id).
 * For each row: s = sigmoid(logits) in fp32; c = s + bias (selection only);
 * experts form n_group contiguous groups of E / n_group; a group scores the
 * sum of its two largest c; the topk_group best groups survive (equal scores:
 * lower group index); ids = the K surviving experts with the largest c, in
 * descending c, equal c to the lower id; weights = s[ids], divided by their
 * sum when norm_topk_prob, then times routed_scaling_factor.
 *   logits  [T, E] fp32      bias [E] fp32 or NULL
 *   ids     [T, K] int32 (written)   weights [T, K] fp32 (written)
 * Errors: INVALID_ARG for NULL logits/ids/weights, T < 0, K < 1, K > E,
 *   n_group < 1, E % n_group != 0, topk_group < 1, topk_group > n_group,
 *   n_group > 1 with E / n_group < 2 (no top-2 group score), or
 *   K > topk_group * E / n_group (too few surviving experts);
 *   UNSUPPORTED for E > MOE_MAX_EXPERTS, K > MOE_MAX_TOPK,
 *   n_group > MOE_MAX_GROUPS.  Non-finite logits: undefined result. */
moe_status moe_route(const float *logits, const float *bias, int T, int E, int K,
                     int n_group, int topk_group, int norm_topk_prob,
                     float routed_scaling_factor, int32_t *ids, float *weights,
                     moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Dispatch: expert-major permutation of the T*K routes.  [M6.1] 0x05A (route
 * row as the reversible unit; rows sorted by (expert, token, slot); offsets
 * [E+1]) and 0x05E (histogram + prefix-sum offsets + packed routes).
 * Route r = t*K + k is token t's k-th choice ids[t, k].
 *   ids       [T, K] int32 in [0, E), distinct within a row
 *   counts    [E] int32 (written): routes per expert
 *   offsets   [E+1] int32 (written): exclusive prefix sum, offsets[E] = T*K;
 *             a zero-hit expert has equal adjacent offsets
 *   route_src [T*K] int32 (written): route held by packed row j, rows of one
 *             expert contiguous, in ascending (token, slot) order
 *   route_pos [T*K] int32 (written): packed row of route r (the inverse)
 *   ws        scratch of moe_dispatch_workspace_size(T, K, E) bytes
 * Errors: INVALID_ARG for NULL pointers, T < 0, K < 1, K > E;
 *   UNSUPPORTED for E > MOE_MAX_EXPERTS, K > MOE_MAX_TOPK; WORKSPACE.
 *   Ids out of range or repeated within a row: undefined result. */
size_t moe_dispatch_workspace_size(int T, int K, int E);
moe_status moe_dispatch(const int32_t *ids, int T, int K, int E,
                        int32_t *counts, int32_t *offsets, int32_t *route_src,
                        int32_t *route_pos, void *ws, size_t ws_bytes,
                        moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Fixed capacity.  [M6.1] 0x06 (C = ceil(CF * T * k / E) slots per expert
 * for the call's routing group), 0x06A (which routes survive: per expert,
 * descending gate, then ascending token, then ascending selected slot; the
 * first C are accepted, the rest overflow), 0x05E (the accepted routes are
 * packed in (expert, token, slot) order), 0x05F (an overflowed route is
 * neither packed nor combined; no renormalisation).
 *
 * moe_capacity_slots: C for a capacity factor (CF > 0, computed as
 *   ceil((double)CF * T * K / E)); -1 for invalid arguments or a C past
 *   INT_MAX.  Host only.
 * moe_dispatch_capacity: as moe_dispatch, for the accepted routes only.
 *   ids [T, K] as moe_dispatch;  weights [T, K] fp32: the gates ranked
 *   counts [E] (written): accepted routes per expert, min(routes, C)
 *   offsets [E+1] (written): prefix sum of counts
 *   route_src [T*K] (the first offsets[E] written): accepted routes in
 *             (expert, token, slot) order
 *   route_pos [T*K] (written): packed row of route r, or -1 if it overflowed
 *   ws        scratch of moe_dispatch_capacity_workspace_size(T, K, E) bytes
 * Errors: as moe_dispatch, plus INVALID_ARG for capacity < 0 or NULL
 *   weights.  Deterministic: no floating-point atomics, the rank order is a
 *   total order. */
int moe_capacity_slots(int T, int K, int E, float capacity_factor);
size_t moe_dispatch_capacity_workspace_size(int T, int K, int E);
moe_status moe_dispatch_capacity(const int32_t *ids, const float *weights, int T, int K, int E,
                                 int capacity, int32_t *counts, int32_t *offsets,
                                 int32_t *route_src, int32_t *route_pos, void *ws, size_t ws_bytes,
                                 moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Routed experts on dispatched rows: for packed row j of expert e (offsets[e]
 * <= j < offsets[e+1]), with token t = route_src[j] / K:
 *   y_packed[j] = W_down_e relu(W_up_e x[t])^2          (no gate, no weight)
 * [circuit] "Routing Is Cheap; Expert Memory Is The Hard Part" (each active
 * expert is a dense ReLU2 MLP); [M6.1] 0x05B (packed expert inputs/outputs);
 * [NemotronH] "Arithmetic" (bf16 path: h = bf16(relu(bf16(W_up x))^2), fp32
 * accumulation).  With route_src == NULL the rows are x[j] themselves
 * (K must be 1): this is how a shared expert runs (E = 1, offsets {0, T}).
 *   x         [T, d_e] in dt;  w_up [E, F, d_e] packed OUT_IN;
 *             w_down_t [E, F, d_e] packed NEURON_MAJOR (moe_pack_weight)
 *   y_packed  [T*K, d_e] in dt (written; rows of experts with no routes untouched)
 *   zero_count int64[2] or NULL: when given, [0] receives the number of exact
 *             zeros in the ReLU^2 activations and [1] the number of hidden
 *             rows of W_down_t the down projection skipped (added to the
 *             current values; the caller clears them).  Needs the decode
 *             path (bf16, MOE_FLAG_ZERO_SKIP_DOWN, T <= 256, d_e <= 4096);
 *             UNSUPPORTED otherwise.
 *   flags     MOE_FLAG_ZERO_SKIP_DOWN or 0
 *   ws        scratch of moe_experts_workspace_size(...) bytes
 * Errors: INVALID_ARG for NULL pointers, T < 0, K < 1, E < 1, F < 1, d_e < 1,
 *   route_src == NULL with K != 1; UNSUPPORTED for d_e or F not a multiple of
 *   8 or pointers not 16-byte aligned; WORKSPACE. */
size_t moe_experts_workspace_size(moe_dtype dt, int T, int d_e, int K, int E, int F, int flags);
moe_status moe_experts(const void *x, moe_dtype dt, int T, int d_e, int K,
                       const int32_t *route_src, const int32_t *offsets, int E, int F,
                       const void *w_up, const void *w_down_t, int flags,
                       void *y_packed, int64_t *zero_count, void *ws, size_t ws_bytes,
                       moe_stream_t stream);

/* moe_experts with FP8 expert weights (MOE_FLAG_FP8_EXPERTS): w_up and
 * w_down_t are E4M3 codes packed with dt MOE_FP8_E4M3, w_up_scale [E, F] and
 * w_down_scale [E, d_e] their fp32 per-output-channel scales; x and y_packed
 * are bf16 (dt must be MOE_BF16).  y_packed[j] = W_down_e relu(W_up_e x[t])^2
 * with W = scale * E4M3 value; the up scale is applied to the fp32 sum
 * before ReLU^2's rounding points, the down scale to the fp32 sum before the
 * output rounding.  Workspace: moe_experts_workspace_size(MOE_BF16, ...).
 * Errors: as moe_experts, plus INVALID_ARG for NULL scales or dt not bf16,
 *   UNSUPPORTED for d_e or F not a multiple of 16. */
moe_status moe_experts_fp8(const void *x, moe_dtype dt, int T, int d_e, int K,
                           const int32_t *route_src, const int32_t *offsets, int E, int F,
                           const void *w_up, const float *w_up_scale, const void *w_down_t,
                           const float *w_down_scale, int flags, void *y_packed,
                           int64_t *zero_count, void *ws, size_t ws_bytes, moe_stream_t stream);

/* moe_experts with MXFP4 expert weights (MOE_FLAG_MXFP4_EXPERTS): w_up
 * [E, F, d_e] codes packed [OUT_IN] with scales w_up_e8 [E, d_e / 32, F];
 * the down projections as codes packed twice, w_down_t [E, F, d_e]
 * NEURON_MAJOR (the decode path) and w_down [E, d_e, F] [OUT_IN] (the
 * grouped GEMMs), with scales w_down_e8 [E, F / 32, d_e]; x and y_packed
 * bf16 (dt must be MOE_BF16).  y_packed[j] = W_down_e relu(W_up_e x[t])^2
 * with W = 2^(e - 127) * E2M1 value.  Workspace:
 * moe_experts_workspace_size(MOE_BF16, ...).
 * Errors: as moe_experts, plus INVALID_ARG for NULL codes or scales or dt
 *   not bf16, UNSUPPORTED for d_e or F not a multiple of 32. */
moe_status moe_experts_mxfp4(const void *x, moe_dtype dt, int T, int d_e, int K,
                             const int32_t *route_src, const int32_t *offsets, int E, int F,
                             const void *w_up, const uint8_t *w_up_e8, const void *w_down_t,
                             const void *w_down, const uint8_t *w_down_e8, int flags,
                             void *y_packed, int64_t *zero_count, void *ws, size_t ws_bytes,
                             moe_stream_t stream);

/* ------------------------------------------------------------------------
 * Weighted combine: out[t] = sum_k w[t,k] * y_packed[route_pos[t*K+k]]
 * (+ y_shared[t]) (+ out[t] with MOE_FLAG_ACCUMULATE_OUT), summed in fp32 in
 * ascending expert id, then the shared row, then the old output, and
 * rounded once.  [M6.1] 0x05B (Y_t = sum of gated packed rows), 0x05E
 * (add, never overwrite), 0x05F (residual kept outside Y); [NemotronH]
 * "Arithmetic" (weighted sum in fp32 in ascending expert id, one rounding).
 *   y_packed [T*K, d] in dt;  weights [T, K] fp32;  ids [T, K] int32
 *   route_pos [T*K] int32 (-1: an overflowed route, skipped);
 *   y_shared [T, d] fp32 or NULL;  out [T, d] in dt
 * Errors: INVALID_ARG for NULL required pointers, T < 0, K < 1, d < 1;
 *   UNSUPPORTED for d % 8 != 0, K > MOE_MAX_TOPK, unaligned pointers. */
moe_status moe_combine(const void *y_packed, const float *weights, const int32_t *ids,
                       const int32_t *route_pos, const float *y_shared, int T, int K,
                       int d, moe_dtype dt, int flags, void *out, moe_stream_t stream);

/* ------------------------------------------------------------------------
 * The fused layer: router logits -> route -> dispatch -> [latent in] ->
 * routed + shared up projections with ReLU^2 -> down projections -> combine
 * -> [latent out] -> out [T, d] in act_dtype.  [circuit] "The Four Layer
 * Kinds CKE Must Preserve" (moe: router, group-limited top-k, routed ReLU2
 * experts + shared expert); [8GB] "The only number that matters" (experts
 * of the latent layer run in the latent width); the steps are the staged
 * calls above.  The router always reads the full-width x.  In a latent layer
 * the combine runs in the latent width, its fp32 sum is rounded to act_dtype,
 * projected back to d, and the shared expert (on the full-width x) is added
 * in that projection's fp32 epilogue.
 *   x [T, d], out [T, d] in act_dtype; ws of moe_workspace_size(desc, T) bytes.
 * Errors: as the staged calls; INVALID_ARG for a NULL desc/weights or a
 *   required weight pointer that is NULL; WORKSPACE. */
size_t moe_workspace_size(const moe_layer_desc *desc, int T);
moe_status moe_layer_forward(const moe_layer_desc *desc, const moe_layer_weights *w,
                             const void *x, int T, void *out, void *ws, size_t ws_bytes,
                             moe_stream_t stream);

/* Where moe_layer_forward leaves the routing it computed, inside the
 * caller's workspace: byte offsets from the start of ws for a call with the
 * same desc and T.  After the call has completed on its stream, ws holds
 *   ids       [T, K] int32   the selected experts of each row, descending
 *                            corrected score, equal scores by lower id
 *   weights   [T, K] fp32    their gate weights (normalised, scaled)
 *   counts    [E]    int32   routes per expert
 *   offsets   [E+1]  int32   exclusive prefix sum of counts
 *   route_src [T*K]  int32   the route (t*K + k) of each packed row, in
 *                            (expert, token, slot) order
 *   route_pos [T*K]  int32   the packed row of each route (-1: a route the
 *                            capacity-bounded variant dropped)
 * on every path the call may take (grouped GEMMs, the decode path, the
 * fused small-batch decode path), as the staged calls moe_route and
 * moe_dispatch (or moe_dispatch_capacity) would return them: the dispatch
 * metadata of [M6.1] 0x05A / 0x05E.  A read-only view for callers that
 * need the layer's own routing (load statistics, auditing the choice).
 * Errors: as moe_workspace_size's checks (INVALID_ARG for NULL out or a
 *   bad desc); T == 0 gives offsets of an empty routing. */
typedef struct {
  size_t ids, weights, counts, offsets, route_src, route_pos;
} moe_routing_layout;
moe_status moe_workspace_routing(const moe_layer_desc *desc, int T, moe_routing_layout *out);

/* moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a static device
 * array of MOE_NOALLOC_SCRATCH_BYTES inside the library: each GPU the
 * library runs on holds one from the library's load until the process
 * ends.  The call itself allocates nothing; x, out and the weights are the
 * caller's, as for moe_layer_forward, and the result is the same.  The
 * array's device address is looked up on the first call on each GPU, which
 * must be the current device and the stream's device.
 * Every call on one GPU shares that GPU's array and overwrites what the
 * last call left in it: calls that overlap on one GPU (other streams,
 * other host threads) race, so the caller orders them (one stream).
 * 64 MiB covers, for the Nano layer (d 2688, 128 experts, top-6, F 1856,
 * shared 3712), decode batches up to 16 rows and grouped-GEMM batches up to
 * 512 rows.
 * Errors: as moe_layer_forward; UNSUPPORTED when moe_workspace_size(desc,
 *   T) exceeds MOE_NOALLOC_SCRATCH_BYTES (nothing is launched); HIP when
 *   the array's address cannot be found. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_layer_forward_noalloc(const moe_layer_desc *desc, const moe_layer_weights *w,
                                     const void *x, int T, void *out, moe_stream_t stream);

/* Stages of moe_layer_forward, for moe_layer_forward_timed. */
enum {
  MOE_STAGE_ROUTER_GEMM = 0,
  MOE_STAGE_ROUTE = 1,
  MOE_STAGE_DISPATCH = 2,
  MOE_STAGE_LATENT_IN = 3,
  MOE_STAGE_UP = 4,
  MOE_STAGE_DOWN = 5,
  MOE_STAGE_COMBINE = 6,
  MOE_STAGE_LATENT_OUT = 7,
  MOE_STAGE_NORM = 8, /* the RMSNorm of MOE_FLAG_PRENORM_RESIDUAL, first */
  MOE_NUM_STAGES = 9
};

/* moe_layer_forward, recording events[2*s] on `stream` before stage s and
 * events[2*s+1] after it (hipEvent_t handles created by the caller; a stage
 * that does not run records both at the same point).  events may be NULL.
 * Used to time each stage's kernels in place. */
moe_status moe_layer_forward_timed(const moe_layer_desc *desc, const moe_layer_weights *w,
                                   const void *x, int T, void *out, void *ws, size_t ws_bytes,
                                   moe_stream_t stream, void *const *events);

/* ------------------------------------------------------------------------
 * Backward pass: the gradients of a loss L through the layer output Y, given
 * dY = dL/dY.  [M6.1] 0x06F (its steps for a softmax router and SwiGLU
 * experts, taken here for the sigmoid router and ReLU^2 experts):
 *  - the forward relation is frozen: the call recomputes the forward's ids,
 *    gates, admissions and route maps from x (the same kernels, so the same
 *    choices), and the experts' h = relu(W_up x)^2 and outputs U;
 *  - combine adjoint (0x06F.2): dU_r = g_r dY_t for an accepted route r =
 *    (t, k), and q_r = <dY_t, U_r> (0 for an overflowed route);
 *  - gate adjoint: with g_k = rsf s_k / sum_j s_j (normalised; otherwise
 *    rsf s_k), dL/ds_k = (rsf q_k - sum_j g_j q_j) / sum_j s_j (resp.
 *    rsf q_k) and dL/dz_k = dL/ds_k s_k (1 - s_k); an overflowed route
 *    still gets -s(1-s) sum_j g_j q_j / sum_j s_j (it stays in the
 *    normaliser, the coupling 0x06F.3 describes); unselected logits and the
 *    selection-only bias get no gradient;
 *  - router projection (0x06F.4): dW_r = G_Z^T x, dx += G_Z W_r;
 *  - experts: dh = dU W_down, du = dh * 2 relu(u), dW_down = dU^T h,
 *    dW_up = du^T x, dx_route = du W_up; the shared expert with dU = dY;
 *  - gather adjoint (0x06F.6): every route's dx row is added to its token's.
 * The residual of R = H + Y is outside the operator (the caller adds dY).
 * Arithmetic: bf16 operands on the bf16 MFMA with fp32 accumulation; the
 * recomputed expert outputs U stay fp32 (q feeds a difference of gate
 * terms); dU and du are rounded to bf16 (the operands of the next
 * products), 2 relu(u) is taken as 2 sqrt(h) (h the forward's bf16 value);
 * q, dz and the router gradients in fp32; every sum in a fixed order.
 * With MOE_FLAG_PRENORM_RESIDUAL (the fused front and back: the layer runs
 * on x = RMSNorm(H) * w_norm and out = Y + H) the call takes the hidden
 * state H as x; the steps above run on the normed rows (recomputed, or left
 * by the training forward) with their gradient kept in fp32, and then
 *  - through the norm, with n = H / rms, r = 1 / rms, dn = dx * w_norm:
 *    dH = dY + (dn - n mean(n dn)) r (dY: the residual's path), rounded to
 *    bf16 into grads->dx, and dw_norm = sum over rows of dx * n (fp32);
 *    the one rounding of the normed rows is taken as the identity.
 * A latent layer (d_latent = L > 0: the router and the shared expert on x,
 * the routed experts on x_lat = x W_lin^T, out = y_lat W_lout^T + y_s; the
 * 8 GB Super write-up, "The only number that matters") differentiates its
 * two projections as linear maps: dy_lat = dY W_lout (rounded to bf16) is
 * the combine's upstream gradient, dW_lout = dY^T y_lat; the experts'
 * input gradients, summed per token into dx_lat [T, L] (rounded to bf16),
 * give dx += dx_lat W_lin and dW_lin = dx_lat^T x; dW_up, dW_down are then
 * [E, F, L] and [E, L, F].
 * Scope: act_dtype MOE_BF16, bf16 experts (no MOE_FLAG_FP8_EXPERTS);
 * dropless or capacity-bounded; d <= 8192 with the fused front.
 *
 * Weights: the forward's (moe_layer_weights) plus the up and down matrices
 * (and a latent layer's two projections) packed a second time,
 * MOE_PACK_NEURON_MAJOR from their PyTorch storage (the reduction of the
 * input-gradient products runs over their rows).  d_e below is d_latent
 * for a latent layer, else d. */
typedef struct {
  const void *w_up_nm;          /* [E, F, d_e] W_up storage, packed NEURON_MAJOR    */
  const void *w_down_nm;        /* [E, d_e, F] W_down storage, packed NEURON_MAJOR  */
  const void *w_up_shared_nm;   /* [F_shared, d] NEURON_MAJOR (NULL: no shared)     */
  const void *w_down_shared_nm; /* [d, F_shared] NEURON_MAJOR                       */
  const void *w_latent_in_nm;   /* [L, d] W_lin storage, NEURON_MAJOR (latent only) */
  const void *w_latent_out_nm;  /* [d, L] W_lout storage, NEURON_MAJOR (latent only) */
} moe_layer_weights_bwd;

/* Gradients written by moe_layer_backward (device memory, every element
 * written; an expert no route reached gets zeros). */
typedef struct {
  void *dx;               /* [T, d] bf16: dL/dx through router and experts (dL/dH
                           * with the fused front, the residual included)      */
  float *dw_router;       /* [E, d] fp32                                       */
  float *dw_up;           /* [E, F, d_e] fp32, PyTorch storage                 */
  float *dw_down;         /* [E, d_e, F] fp32, PyTorch storage                 */
  float *dw_up_shared;    /* [F_shared, d] fp32 (unused when F_shared is 0)    */
  float *dw_down_shared;  /* [d, F_shared] fp32                                */
  float *dw_norm;         /* [d] fp32, with MOE_FLAG_PRENORM_RESIDUAL (else unused) */
  float *dw_latent_in;    /* [L, d] fp32, latent layer (else unused)           */
  float *dw_latent_out;   /* [d, L] fp32, latent layer (else unused)           */
} moe_layer_grads;

/* x, dy [T, d] bf16.  Errors: as moe_layer_forward, plus UNSUPPORTED outside
 * the scope above; INVALID_ARG for NULL gradient or backward-weight
 * pointers. */
size_t moe_backward_workspace_size(const moe_layer_desc *desc, int T);
moe_status moe_layer_backward(const moe_layer_desc *desc, const moe_layer_weights *w,
                              const moe_layer_weights_bwd *wb, const void *x, const void *dy, int T,
                              const moe_layer_grads *grads, void *ws, size_t ws_bytes,
                              moe_stream_t stream);

/* Training forward: the layer output of moe_layer_forward (within the
 * bf16 bar: here the routed outputs stay fp32 up to the combine's single
 * rounding) computed into the backward's workspace, which then holds the
 * forward state the backward needs (ids, gates, route maps, h, U).
 * moe_layer_backward_saved with the same desc, weights, x, T and workspace
 * (nothing else run on that workspace in between) skips the backward's
 * recomputation of the forward; its gradients are bitwise those of
 * moe_layer_backward.  [M6.1] 0x06F.7 ("saved or recomputed": the same
 * ids and gates either way).  Scope and errors as moe_layer_backward. */
moe_status moe_layer_forward_train(const moe_layer_desc *desc, const moe_layer_weights *w,
                                   const void *x, int T, void *out, void *ws, size_t ws_bytes,
                                   moe_stream_t stream);
moe_status moe_layer_backward_saved(const moe_layer_desc *desc, const moe_layer_weights *w,
                                    const moe_layer_weights_bwd *wb, const void *x, const void *dy,
                                    int T, const moe_layer_grads *grads, void *ws, size_t ws_bytes,
                                    moe_stream_t stream);

/* Phases of moe_layer_backward, for moe_layer_backward_timed. */
enum {
  MOE_BWD_STAGE_FORWARD = 0, /* router, route, dispatch, up and down GEMMs   */
  MOE_BWD_STAGE_GATES = 1,   /* combine and gate adjoints, router gradient   */
  MOE_BWD_STAGE_DH = 2,      /* dh = dU W_down with the ReLU^2 derivative     */
  MOE_BWD_STAGE_DX = 3,      /* dx rows = du W_up, the per-token sum          */
  MOE_BWD_STAGE_TRANSPOSE = 4, /* the weight-gradient operands, transposed    */
  MOE_BWD_STAGE_DW_DOWN = 5, /* dW_down = dU^T h per expert (+ shared)        */
  MOE_BWD_STAGE_DW_UP = 6,   /* dW_up = du^T x per expert (+ shared)          */
  MOE_BWD_NUM_STAGES = 7
};

/* moe_layer_backward (saved = 0) or moe_layer_backward_saved (saved = 1)
 * recording events[2*s] / events[2*s+1] around phase s on `stream`
 * (hipEvent_t handles created by the caller), or none when events is NULL;
 * a phase that does not run records both at the same point. */
moe_status moe_layer_backward_timed(const moe_layer_desc *desc, const moe_layer_weights *w,
                                    const moe_layer_weights_bwd *wb, const void *x, const void *dy,
                                    int T, const moe_layer_grads *grads, void *ws, size_t ws_bytes,
                                    moe_stream_t stream, void *const *events, int saved);

/* Name of a status code (a static string). */
const char *moe_status_string(moe_status st);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
