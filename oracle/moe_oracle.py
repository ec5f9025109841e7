"""CPU oracle for the routed ReLU^2 MoE layer forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header,
helper, table or constant with the HIP library and imports nothing from it.

It is the plain definition of the layer, computed slowly in float64 with
numpy.  A library matmul is the only primitive used; there is no blocking,
fusion or reordering beyond what the definition states.  Every function names
the passage of the source pages it follows:

* [Nemotron circuit]  "Nemotron is not one circuit: Mamba, attention and MoE
  routing" (shivasnotes.com), sections "The Four Layer Kinds CKE Must
  Preserve", "The Router Is A Deterministic Algorithm", "The C Kernel
  Contract", "Routing Is Cheap; Expert Memory Is The Hard Part".
* [M6.1]  "M6.1 - Routed Capacity: MoE Experts, Routers, and Token Dispatch"
  (transformer-system.numinens.com), sections 0x01E, 0x04A, 0x05A-0x05F.
* [NemotronH]  "NemotronH (Nemotron 3.5 Lightning, Bolt, Super VL)"
  (tandemllm docs v0.13.0), section "Arithmetic".
* [8 GB Super]  the hot.atechcom.net write-up of Nemotron-3.5-Super on an
  8 GB card, sections "The only number that matters: bytes per token" and
  "The engine, step by step" (item 4, skipping zeros).
* [Nemotron circuit] "The Four Layer Kinds CKE Must Preserve" also places
  the layer between an RMSNorm and a residual add; [NemotronH]
  "Arithmetic" fixes that norm to fp32 times the plain weight; [M6.1]
  0x06F.1 writes the residual outside the MoE operator, ``R_t = H_t + Y_t``.

Precision.  Every floating-point result is float64 with no intermediate
rounding, with two exceptions.  The optional RMSNorm in front of the layer
is the float64 definition rounded once to the activation dtype (that
rounding makes the layer's input values; see ``rms_norm``).  The other is
where floating point decides a discrete value, the router's selection: the pages fix the router precision to fp32 (fp32 logits, sigmoid; [NemotronH] "Arithmetic"), so the selection is
taken on fp32-rounded scores ``s32 = fp32(sigmoid(z))`` and
``c32 = fp32(s32 + b)``, and on fp32 group sums.  The gate *weights* are
computed in float64 from the unrounded sigmoid.

Pins.  Each function here is pinned by ``tests/test_oracle_pins.py`` against
values the pages print, closed forms, brute force on tiny inputs and
algebraic identities; see the docstrings for what pins what.  The
zero-fraction diagnostic (``relu2_zero_fraction``) has no page value; it is
pinned by closed forms on hand-made rows.
"""
from __future__ import annotations

import math

import numpy as np

f64 = np.float64
f32 = np.float32


# ---------------------------------------------------------------------------
# RMSNorm in front of the layer
# ---------------------------------------------------------------------------

def round_to_act(a32, act_dtype):
    """Round fp32 values to the activation dtype: bfloat16 (the upper 16
    bits of binary32) by round-to-nearest-even, or fp32 unchanged.  Returned
    as float64 holding the rounded values exactly.  The input is taken as
    fp32 first (used for values that are already fp32)."""
    a32 = np.asarray(a32, dtype=f32)
    if act_dtype == "f32":
        return a32.astype(f64)
    u = a32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(f32).astype(f64)


def round_once(v, act_dtype):
    """Round float64 values once, to nearest with ties to even, to the
    activation dtype (bfloat16: 8 significant bits, the exponent range of
    binary32; or fp32).  No intermediate fp32 rounding, so a value just
    above a bfloat16 midpoint rounds up even when fp32 would first have
    rounded it onto the midpoint.  Returned as float64."""
    v = np.asarray(v, dtype=f64)
    if act_dtype == "f64":                  # no rounding (central-difference checks of gradients)
        return v
    if act_dtype == "f32":
        return v.astype(f32).astype(f64)
    m, e = np.frexp(v)                      # v = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                 # below 2^-126 the spacing stays 2^-133
    q = np.ldexp(1.0, e - 8)                # spacing of bfloat16 values near v
    r = np.rint(v / q) * q                  # np.rint: ties to even
    big = np.abs(r) > float(np.ldexp(255.0 / 128.0, 127))
    return np.where(big, np.copysign(np.inf, v), r)


def rms_norm_exact(h, w_norm, eps):
    """``h / sqrt(mean(h^2) + eps) * w`` per row, in float64, unrounded.

    [NemotronH] "Arithmetic": the RMS norm multiplies by the plain weight
    (not 1 + w); [Nemotron circuit] "The Four Layer Kinds CKE Must
    Preserve": the MoE layer's input is the RMSNorm of the hidden state.
    The mean is over the row's width; eps is added under the root."""
    h = np.asarray(h, dtype=f64)
    w = np.asarray(w_norm, dtype=f64)
    ms = np.mean(h * h, axis=1)
    return h / np.sqrt(ms + float(eps))[:, None] * w[None, :]


def rms_norm_backward(h, w_norm, eps, dx):
    """Gradients through ``x = n * w``, ``n = h / r``, ``r = sqrt(mean(h^2)
    + eps)`` (``rms_norm_exact``), in float64, given ``dx = dL/dx`` [T, d].
    With ``dn = dx * w`` and ``d n_i / d h_j = (delta_ij - n_i n_j / d) / r``
    (the mean is over the width d): ``dh = (dn - n * mean(n * dn)) / r``;
    ``dw = sum over rows of dx * n``.  Returns (dh [T, d], dw [d])."""
    h = np.asarray(h, dtype=f64)
    w = np.asarray(w_norm, dtype=f64)
    dx = np.asarray(dx, dtype=f64)
    r = np.sqrt(np.mean(h * h, axis=1) + float(eps))[:, None]
    n = h / r
    dn = dx * w[None, :]
    dh = (dn - n * np.mean(n * dn, axis=1, keepdims=True)) / r
    return dh, (dx * n).sum(axis=0)


def rms_norm(h, w_norm, eps, act_dtype):
    """The RMSNorm of each row (``rms_norm_exact``), rounded once to the
    activation dtype.  [NemotronH] "Arithmetic" fixes the norm's precision
    to fp32; the definition is evaluated here in float64, which is at least
    as accurate, and rounded once at the end, so any fp32 evaluation differs
    from it only through its own rounding error (the bound a GPU result is
    held to)."""
    return round_once(rms_norm_exact(h, w_norm, eps), act_dtype)


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------

def router_logits(x, w_router):
    """Router logits ``z = x . W_r^T`` with the router stored as [E, d].

    [M6.1] 0x04A: a PyTorch ``nn.Linear(d, E)`` stores its weight as
    [out, in] = [E, d], so the runtime equation is ``Z = H W_stored^T``.
    """
    return np.asarray(x, dtype=f64) @ np.asarray(w_router, dtype=f64).T


def sigmoid(z):
    """Sigmoid router probabilities ([Nemotron circuit] "The Router Is A
    Deterministic Algorithm": the group-limited router receives sigmoid
    probabilities; [NemotronH] "Arithmetic": fp32 logits, sigmoid)."""
    z = np.asarray(z, dtype=f64)
    return 1.0 / (1.0 + np.exp(-z))


def decision_scores(logits, bias):
    """Scores the router chooses with.

    Returns ``(s64, s32, c32, c64)``: the sigmoid in float64, the sigmoid
    rounded to fp32, the bias-corrected selection score ``c = s + b`` in fp32
    (one fp32 add of the fp32 sigmoid and the fp32 bias), and the same
    corrected score in float64 (used only to measure how close a row is to a
    tie).  The correction bias affects only the selection score
    ([Nemotron circuit] "The Router Is A Deterministic Algorithm";
    [NemotronH] "Arithmetic": the bias is for the choice only).  A missing
    bias is zero.
    """
    s64 = sigmoid(logits)
    E = s64.shape[-1]
    b32 = np.zeros(E, dtype=f32) if bias is None else np.asarray(bias, dtype=f32)
    s32 = s64.astype(f32)
    c32 = (s32 + b32).astype(f32)
    c64 = s64 + b32.astype(f64)
    return s64, s32, c32, c64


def group_scores(c, n_group):
    """Score of each expert group: the sum of its two largest corrected
    scores ([Nemotron circuit] "The Router Is A Deterministic Algorithm":
    experts are split into equal groups, a group's score is the sum of its
    two largest corrected expert scores).  Groups are contiguous id blocks of
    ``E / n_group`` experts.  The sum is taken in the dtype of ``c`` (fp32 for
    the decision)."""
    T, E = c.shape
    g = c.reshape(T, n_group, E // n_group)
    top2 = -np.sort(-g, axis=-1)[..., :2]
    return (top2[..., 0] + top2[..., 1]).astype(c.dtype)


def eligible_experts(c32, n_group, topk_group):
    """Boolean [T, E] mask of experts that survive group selection.

    The router keeps the ``topk_group`` best groups and masks every other
    group ([Nemotron circuit] "The Router Is A Deterministic Algorithm").
    Equal group scores are broken toward the lower group index (the pages'
    lower-id rule for experts, extended to groups).  Masked experts can never
    be selected.  With ``n_group == 1`` every expert is eligible.
    """
    T, E = c32.shape
    if n_group == 1:
        return np.ones((T, E), dtype=bool)
    G = group_scores(c32, n_group)
    # stable sort of -G: equal scores keep ascending group order
    order = np.argsort(-G, axis=1, kind="stable")
    keep = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(keep, order[:, :topk_group], True, axis=1)
    return np.repeat(keep, E // n_group, axis=1)


def select_experts(c32, eligible, K):
    """Global top-K of the surviving corrected scores, in descending score;
    equal scores go to the lower expert id ([Nemotron circuit] "The Router Is
    A Deterministic Algorithm" and "The C Kernel Contract": a deterministic
    expert-index tie break; [NemotronH] "Arithmetic": ties to the lower id)."""
    key = np.where(eligible, -c32.astype(f64), np.inf)
    order = np.argsort(key, axis=1, kind="stable")
    return order[:, :K].astype(np.int32)


def gate_weights(s64, ids, norm_topk_prob, routed_scaling_factor):
    """Output weights: gathered from the *uncorrected* sigmoid scores,
    normalised over the selected experts if configured, then multiplied by
    the routed scaling factor ([Nemotron circuit] "The Router Is A
    Deterministic Algorithm").  The normalisation has no epsilon: a sum of
    K >= 1 sigmoids is positive.  Scaling is applied whether or not the
    weights were normalised."""
    w = np.take_along_axis(s64, ids.astype(np.int64), axis=1)
    if norm_topk_prob:
        w = w / w.sum(axis=1, keepdims=True)
    return w * float(routed_scaling_factor)


def route(logits, bias, n_group, topk_group, K, norm_topk_prob, routed_scaling_factor):
    """The group-limited sigmoid router for every row of ``logits`` [T, E].

    Follows the order of [Nemotron circuit] "The Router Is A Deterministic
    Algorithm": sigmoid, corrected score, group scores, keep the best groups,
    global top-K of the survivors, gather the uncorrected scores, normalise,
    scale.  Returns ``ids`` [T, K] int32 (descending corrected score, ties to
    the lower id) and ``weights`` [T, K] float64, plus ``info`` with the
    float64 boundary gap of each row (how far the row is from changing its
    choice) and whether the expert boundary is an exact tie of bitwise-equal
    inputs.
    """
    logits = np.asarray(logits, dtype=f64)
    T, E = logits.shape
    s64, s32, c32, c64 = decision_scores(logits, bias)
    elig = eligible_experts(c32, n_group, topk_group)
    ids = select_experts(c32, elig, K)
    w = gate_weights(s64, ids, norm_topk_prob, routed_scaling_factor)
    info = _boundary_info(logits, bias, c32, c64, elig, ids, n_group, topk_group, K)
    return ids, w, info


def _boundary_info(logits, bias, c32, c64, elig, ids, n_group, topk_group, K):
    """Distance of each row from a different choice (float64).

    ``gap`` = min(K-th minus (K+1)-th eligible corrected score, and with
    groups the topk_group-th minus next group score).  ``exact_tie`` marks
    rows whose K-th and (K+1)-th eligible experts (in fp32 decision order)
    have bitwise-equal logits and bias, so any implementation sees a tie.
    """
    T, E = c64.shape
    gap = np.full(T, np.inf)
    n_elig = elig.sum(axis=1)
    c64m = np.where(elig, c64, -np.inf)
    srt = -np.sort(-c64m, axis=1)
    has_next = n_elig > K
    if K < E:
        gap[has_next] = (srt[has_next, K - 1] - srt[has_next, K])
    if n_group > 1 and topk_group < n_group:
        G = -np.sort(-group_scores(c64, n_group), axis=1)
        gap = np.minimum(gap, G[:, topk_group - 1] - G[:, topk_group])
    exact_tie = np.zeros(T, dtype=bool)
    key = np.where(elig, -c32.astype(f64), np.inf)
    order = np.argsort(key, axis=1, kind="stable")
    b = np.zeros(E, dtype=f32) if bias is None else np.asarray(bias, dtype=f32)
    z32 = logits.astype(f32)
    for t in np.nonzero(has_next)[0]:
        i, j = order[t, K - 1], order[t, K]
        if c32[t, i] == c32[t, j] and z32[t, i] == z32[t, j] and b[i] == b[j]:
            exact_tie[t] = True
    return {"gap": gap, "exact_tie": exact_tie}


# ---------------------------------------------------------------------------
# Dispatch
# ---------------------------------------------------------------------------

def dispatch(ids, E):
    """Expert-major dispatch metadata for the accepted routes.

    Route ``r = t*K + k`` is token ``t``'s ``k``-th selection.  Following
    [M6.1] 0x05A (route row as the reversible unit) and 0x05E (count,
    prefix-sum offsets, packed expert-major routes):

    * ``counts[e]`` = routes that selected expert ``e``;
    * ``offsets`` = exclusive prefix sum, ``offsets[E] = T*K``; a zero-hit
      expert has equal adjacent offsets ([M6.1] 0x05F);
    * ``route_src[j]`` = the route in packed row ``j``, routes sorted by
      (expert, token, slot) -- the deterministic teaching layout of 0x05A;
    * ``route_pos[r]`` = the packed row of route ``r`` (inverse permutation).
    """
    ids = np.asarray(ids)
    T, K = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    tok = np.repeat(np.arange(T), K)
    slot = np.tile(np.arange(K), T)
    route_src = np.lexsort((slot, tok, flat)).astype(np.int32)  # last key is primary
    route_pos = np.empty(T * K, dtype=np.int32)
    route_pos[route_src] = np.arange(T * K, dtype=np.int32)
    return counts, offsets, route_src, route_pos


# ---------------------------------------------------------------------------
# Fixed capacity (the capacity-bounded variant of dispatch)
# ---------------------------------------------------------------------------

def capacity_slots(T, K, E, capacity_factor):
    """Route slots per expert for one routing group, ``C = ceil(CF * T * k /
    E)`` ([M6.1] 0x06 "Expert Capacity And Overflow").  The routing group is
    the call's T rows.  CF is taken as an fp32 value (the layer description
    carries it in fp32) and ``(CF * T * k) / E`` is evaluated in float64."""
    return int(math.ceil(float(np.float32(capacity_factor)) * T * K / E))


def arbitrate_capacity(ids, gates, C):
    """Which routes fit under a capacity of C slots per expert.

    [M6.1] 0x06A "Overflow Requires An Arbitration Order": each expert's
    routes are ranked by descending gate, then ascending token id, then
    ascending selected slot; the first C are accepted and the rest overflow.
    Returns ``(accept [T, K] bool, gap [E])`` where ``gap[e]`` is the gate of
    expert e's last accepted route minus that of its first overflowed route
    (inf when nothing overflows): how close the decision was.
    """
    ids = np.asarray(ids)
    gates = np.asarray(gates, dtype=f64)
    T, K = ids.shape
    accept = np.zeros((T, K), dtype=bool)
    E = int(ids.max()) + 1 if ids.size else 0
    gap = np.full(max(E, 1), np.inf)
    for e in range(E):
        tt, ss = np.nonzero(ids == e)
        routes = sorted(zip(tt.tolist(), ss.tolist()), key=lambda r: (-gates[r[0], r[1]], r[0], r[1]))
        for t, k in routes[:C]:
            accept[t, k] = True
        if C < len(routes):
            a, b = routes[C - 1] if C > 0 else None, routes[C]
            gap[e] = (gates[a] - gates[b]) if a is not None else np.inf
    return accept, gap


def dispatch_accepted(ids, accept, E):
    """``dispatch`` over the accepted routes only: packed rows in (expert,
    token, slot) order ([M6.1] 0x05E, ``dispatch_accepted_routes``), counts
    and offsets of the accepted routes, and ``route_pos[r] = -1`` for a route
    that overflowed (it is neither packed nor combined; [M6.1] 0x05F)."""
    ids = np.asarray(ids)
    T, K = ids.shape
    acc = np.asarray(accept).reshape(-1)
    flat = ids.reshape(-1).astype(np.int64)
    counts = np.bincount(flat[acc], minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    tok = np.repeat(np.arange(T), K)
    slot = np.tile(np.arange(K), T)
    order = np.lexsort((slot, tok, flat))
    route_src = order[acc[order]].astype(np.int32)
    route_pos = np.full(T * K, -1, dtype=np.int32)
    route_pos[route_src] = np.arange(len(route_src), dtype=np.int32)
    return counts, offsets, route_src, route_pos


# ---------------------------------------------------------------------------
# FP8 expert weights (the low-precision variant)
# ---------------------------------------------------------------------------
#
# [NemotronH] "How the engine runs it" and [8 GB Super] run the experts from
# low-precision checkpoints (FP8 and 4-bit formats with shared scales).  The
# format used here is the OCP 8-bit floating point E4M3 (the "FN" variant:
# 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no infinities,
# S.1111.111 the only NaN, largest finite value 448), one fp32 scale per
# output channel (per row of the [out, in] weight).  Activations stay in the
# activation dtype; the weights are used as scale * value, exactly.

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Values of E4M3 codes (uint8) as float64: exponent field 0 is
    subnormal, m / 8 * 2^-6; otherwise (1 + m / 8) * 2^(e - 7); 0x7F / 0xFF
    are NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e4m3_encode(v):
    """The E4M3 code nearest to each fp32 value, ties to the even code
    (round-to-nearest-even on the 3-bit mantissa, subnormals included);
    magnitudes past 448 saturate to 448.  -0 keeps its sign bit."""
    v = np.asarray(v, dtype=f32).astype(f64)
    neg = np.signbit(v)
    a = np.abs(v)
    # the quantum of a's binade: 2^(e - 3), e = max(floor(log2 a), -6)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    q = np.exp2(e - 3.0)
    r = np.rint(a / q) * q  # rint: round half to even, exact in float64
    r = np.minimum(r, E4M3_MAX)
    # value -> fields
    er = np.floor(np.log2(np.where(r > 0, r, 1.0)))
    sub = r < 2.0 ** -6
    e_field = np.where(sub, 0, er + 7).astype(np.int64)
    m_field = np.where(sub, np.rint(r / 2.0 ** -9), np.rint((r / np.exp2(er) - 1.0) * 8)).astype(np.int64)
    code = (e_field << 3) | m_field
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_rows_fp8(w):
    """Per-row (per output channel) FP8 quantisation of [..., R, C] weights
    in [out, in] storage: ``s = fp32(amax_row / 448)`` (1 for an all-zero
    row) and ``codes = e4m3_encode(fp32(w / s))``, every step in fp32, so
    each row's largest magnitude lands on 448.  Returns (codes uint8
    [..., R, C], scales fp32 [..., R])."""
    w32 = np.asarray(w, dtype=f64).astype(f32)
    amax = np.max(np.abs(w32), axis=-1)
    s = np.where(amax > 0, amax / f32(E4M3_MAX), f32(1.0)).astype(f32)
    codes = e4m3_encode(w32 / s[..., None])
    return codes, s


def dequant_rows_fp8(codes, scales):
    """``scale * value`` per row, exact in float64."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=f32).astype(f64)[..., None]


def fp8_expert_weights(w):
    """The weight dict with every routed and shared expert matrix replaced by
    its FP8 quantisation, dequantised (what the FP8 layer computes with)."""
    out = dict(w)
    for k in ("w_up", "w_down", "w_up_shared", "w_down_shared"):
        if k in w and w[k] is not None:
            if k in ("w_up", "w_down") and not isinstance(w[k], np.ndarray):
                out[k] = _LazyDequant(w[k])
            else:
                out[k] = dequant_rows_fp8(*quantize_rows_fp8(w[k]))
    return out


class _LazyDequant:
    """Per-expert quantise-dequantise (FP8 unless another round trip is
    given) of a lazily converted [E, ...] weight."""

    def __init__(self, src, roundtrip=None):
        self.src = src
        self.roundtrip = roundtrip
        self.cache = {}

    def __len__(self):
        return len(self.src)

    def __getitem__(self, e):
        e = int(e)
        if e in self.cache:
            return self.cache[e]
        w = self.src[e]
        q = self.roundtrip(w) if self.roundtrip else dequant_rows_fp8(*quantize_rows_fp8(w))
        if getattr(self.src, "cache", True):  # an uncached source stays uncached
            self.cache[e] = q
        return q


# ---------------------------------------------------------------------------
# MXFP4 expert weights (the 4-bit variant)
# ---------------------------------------------------------------------------
#
# [8 GB Super] "The only number that matters: bytes per token" and
# [NemotronH] "How the engine runs it" serve the experts from 4-bit
# checkpoints whose elements share a scale per small block.  The 4-bit
# format used here is MXFP4 of the OCP Microscaling Formats specification
# (v1.0): elements in FP4 E2M1 (1 sign bit, 2 exponent bits with bias 1, 1
# mantissa bit, no infinities or NaN: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4,
# 6), a block of 32 consecutive elements along the reduction (input)
# dimension sharing one E8M0 scale 2^(e - 127).  The shared exponent of a
# block is floor(log2(amax)) - 2 (2 being the largest E2M1 exponent),
# clamped to the E8M0 range [-127, 127]; each element is then v / 2^shared
# rounded to E2M1 (nearest, ties to the even code) with magnitudes past 6
# saturating to 6.  An all-zero block takes scale code 0.  Activations stay
# in the activation dtype; the weights are used as scale * value, exactly.

MX_BLOCK = 32
E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes):
    """Values of E2M1 codes (0..15) as float64: bit 3 the sign, bits 2..1 the
    exponent (bias 1; field 0 subnormal, m / 2), bit 0 the mantissa."""
    c = np.asarray(codes).astype(np.int64)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(c & 8, -mag, mag)


def e2m1_encode(v):
    """The E2M1 code nearest to each float64 value, ties to the even code
    (round-to-nearest-even on the 1-bit mantissa); magnitudes past 6
    saturate to 6.  -0 keeps its sign bit."""
    v = np.asarray(v, dtype=f64)
    neg = np.signbit(v)
    a = np.abs(v)
    # the quantum of a's binade: 2^(e - 1), e = max(floor(log2 a), 0)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, 0.0)
    r = np.minimum(np.rint(a / np.exp2(e - 1.0)) * np.exp2(e - 1.0), 6.0)
    mag_code = np.searchsorted(E2M1_MAGS, r)  # r is one of the 8 magnitudes
    return (mag_code | np.where(neg, 8, 0)).astype(np.uint8)


def quantize_blocks_mxfp4(w):
    """MXFP4 quantisation of [..., R, C] weights in [out, in] storage, blocks
    of 32 along C (C a multiple of 32).  Per block: amax in fp32,
    shared = clamp(floor(log2 amax) - 2, -127, 127) (an all-zero block:
    -127), codes = e2m1_encode(w / 2^shared).  Returns (codes uint8 [...,
    R, C], one 4-bit code per element; scales uint8 [..., R, C / 32], the
    E8M0 codes shared + 127)."""
    w32 = np.asarray(w, dtype=f64).astype(f32).astype(f64)
    shp = w32.shape
    assert shp[-1] % MX_BLOCK == 0
    blk = w32.reshape(shp[:-1] + (shp[-1] // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blk), axis=-1)
    with np.errstate(divide="ignore"):
        lg = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
    shared = np.where(amax > 0, np.clip(lg - 2.0, -127.0, 127.0), -127.0)
    codes = e2m1_encode(blk / np.exp2(shared)[..., None]).reshape(shp)
    return codes, (shared + 127).astype(np.uint8)


def dequant_blocks_mxfp4(codes, scales):
    """``2^(scale - 127) * value`` per element, exact in float64."""
    c = np.asarray(codes)
    x = np.exp2(np.asarray(scales, dtype=f64) - 127.0)
    v = e2m1_decode(c).reshape(c.shape[:-1] + (c.shape[-1] // MX_BLOCK, MX_BLOCK))
    return (v * x[..., None]).reshape(c.shape)


def _mxfp4_roundtrip(w):
    return dequant_blocks_mxfp4(*quantize_blocks_mxfp4(w))


def mxfp4_expert_weights(w):
    """The weight dict with every routed and shared expert matrix replaced by
    its MXFP4 quantisation, dequantised (what the MXFP4 layer computes
    with).  Blocks run along each matrix's input dimension: the model width
    for the up projections, the hidden neurons for the down projections."""
    out = dict(w)
    for k in ("w_up", "w_down", "w_up_shared", "w_down_shared"):
        if k in w and w[k] is not None:
            if k in ("w_up", "w_down") and not isinstance(w[k], np.ndarray):
                out[k] = _LazyDequant(w[k], _mxfp4_roundtrip)
            else:
                out[k] = _mxfp4_roundtrip(w[k])
    return out


# ---------------------------------------------------------------------------
# MXFP8 activations (the W4A8 variant: MXFP4 weights, MXFP8 activations)
# ---------------------------------------------------------------------------
#
# The inputs of both expert products -- the rows an up projection reads and
# the ReLU^2 output a down projection reads -- are quantised to MXFP8 of the
# OCP Microscaling Formats specification (v1.0): E4M3 elements sharing one
# E8M0 scale 2^(e - 127) per block of 32 consecutive values along the
# product's reduction dimension.  The shared exponent of a block is
# floor(log2(amax)) - 8 (8 being the largest E4M3 exponent), clamped to
# [-127, 127]; each value is v / 2^shared rounded to E4M3 (nearest, ties to
# even; magnitudes past 448 saturate).  An all-zero block takes scale code
# 0.  The decision is taken on the values the layer holds at that point: an
# up product's input rows in the activation dtype (the model-width rows are
# bf16 already; a latent layer's rows are its projection rounded once to the
# activation dtype), the ReLU^2 output in fp32 (the precision the GPU
# squares it in).  Weights are MXFP4 as above; both operands are used as
# scale * value, exactly; products accumulate in float64 here.

MXFP8_EMAX = 8


def quantize_blocks_mxfp8(a):
    """MXFP8 quantisation of [..., C] values, blocks of 32 along the last
    axis (C a multiple of 32), decided on their fp32 values.  Returns
    (codes uint8 [..., C] E4M3, scales uint8 [..., C / 32] E8M0)."""
    a32 = np.asarray(a, dtype=f64).astype(f32).astype(f64)
    shp = a32.shape
    assert shp[-1] % MX_BLOCK == 0
    blk = a32.reshape(shp[:-1] + (shp[-1] // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blk), axis=-1)
    with np.errstate(divide="ignore"):
        lg = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
    shared = np.where(amax > 0, np.clip(lg - MXFP8_EMAX, -127.0, 127.0), -127.0)
    codes = e4m3_encode(blk / np.exp2(shared)[..., None]).reshape(shp)
    return codes, (shared + 127).astype(np.uint8)


def dequant_blocks_mxfp8(codes, scales):
    """``2^(scale - 127) * value`` per element, exact in float64."""
    c = np.asarray(codes)
    x = np.exp2(np.asarray(scales, dtype=f64) - 127.0)
    v = e4m3_decode(c).reshape(c.shape[:-1] + (c.shape[-1] // MX_BLOCK, MX_BLOCK))
    return (v * x[..., None]).reshape(c.shape)


def mxfp8_roundtrip(a):
    """The values an MXFP8 operand carries: quantise, then dequantise."""
    return dequant_blocks_mxfp8(*quantize_blocks_mxfp8(a))


def activation_quantiser(expert_dtype, act_dtype="bf16"):
    """What the expert products do to their inputs, for the W4A8 variant
    ("mxfp4_a8"): ``aq(v, "in")`` rounds an up product's input rows once to
    the activation dtype and takes their MXFP8 round trip, ``aq(v,
    "hidden")`` the ReLU^2 output's round trip (decided on fp32).  None for
    the other variants."""
    if expert_dtype != "mxfp4_a8":
        return None

    def aq(v, which):
        if which == "in":
            v = round_once(v, act_dtype)
        return mxfp8_roundtrip(v)
    return aq


def quantised_expert_weights(w, expert_dtype):
    """The weights a layer with ``expert_dtype`` ("fp8", "mxfp4",
    "mxfp4_a8" or None / "bf16") computes with."""
    if expert_dtype == "fp8":
        return fp8_expert_weights(w)
    if expert_dtype in ("mxfp4", "mxfp4_a8"):
        return mxfp4_expert_weights(w)
    return w


# ---------------------------------------------------------------------------
# Experts
# ---------------------------------------------------------------------------

def relu2(u):
    """Squared ReLU, ``max(u, 0)^2`` ([Nemotron circuit] "The Four Layer
    Kinds CKE Must Preserve": up projection, ReLU2, down projection)."""
    r = np.maximum(np.asarray(u, dtype=f64), 0.0)
    return r * r


def expert_mlp(x_rows, w_up_e, w_down_e, act_q=None):
    """One routed ReLU^2 expert, no gate: ``W_down relu(W_up x)^2``.

    [M6.1] 0x01E (an expert is ``W_down phi(W_up x)``), with phi = ReLU^2
    ([Nemotron circuit] "Routing Is Cheap; Expert Memory Is The Hard Part";
    [NemotronH] "Arithmetic").  Weights in PyTorch storage order
    ([M6.1] 0x02A): ``w_up_e`` [F, d_e], ``w_down_e`` [d_e, F].  ``act_q``:
    what each product does to its input rows (the W4A8 variant's MXFP8
    round trip), or None.
    """
    x_rows = np.asarray(x_rows, dtype=f64)
    if act_q is not None:
        x_rows = act_q(x_rows, "in")
    h = relu2(x_rows @ np.asarray(w_up_e, dtype=f64).T)
    if act_q is not None:
        h = act_q(h, "hidden")
    return h @ np.asarray(w_down_e, dtype=f64).T


def run_experts(x_e, route_src, offsets, K, w_up, w_down, act_q=None):
    """Run every expert on its packed rows (expert-major batching:
    [Nemotron circuit] "Routing Is Cheap; Expert Memory Is The Hard Part").
    Packed row ``j`` of expert ``e`` carries token ``route_src[j] // K``.
    Returns ``y_packed`` [T*K, d_e] float64 in packed order."""
    x_e = np.asarray(x_e, dtype=f64)
    R = len(route_src)
    y = np.zeros((R, x_e.shape[1]), dtype=f64)
    E = len(offsets) - 1
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        rows = np.asarray(route_src[a:b]) // K
        y[a:b] = expert_mlp(x_e[rows], w_up[e], w_down[e], act_q)
    return y


def shared_expert(x, w_up_s, w_down_s, act_q=None):
    """The shared expert: a dense ReLU^2 MLP on every row, always active,
    ungated and not scaled by the routed scaling factor ([Nemotron circuit]
    "The Four Layer Kinds CKE Must Preserve": routed ReLU2 experts plus a
    shared expert)."""
    return expert_mlp(x, w_up_s, w_down_s, act_q)


def combine(y_packed, weights, ids, route_pos, y_shared=None, out_prev=None):
    """Weighted scatter-combine back to token rows.

    ``Y[t] = sum_k w[t,k] * y_packed[route_pos[t,k]]`` -- an add, never an
    overwrite, over the token's routes ([M6.1] 0x05B packed form, 0x05E
    index_add_ semantics).  Summed in ascending expert id ([NemotronH]
    "Arithmetic": the weighted sum in ascending expert id).  The shared
    expert output is added after the routed sum.  The outer residual is not
    part of the MoE output ([M6.1] 0x05F); it is added only when the caller
    passes ``out_prev`` (the accumulate-into-output mode).  A route with
    ``route_pos = -1`` overflowed a fixed capacity and contributes nothing;
    the token's other gates are not renormalised ([M6.1] 0x05F, fixed-drop
    semantics).
    """
    y_packed = np.asarray(y_packed, dtype=f64)
    ids = np.asarray(ids)
    T, K = ids.shape
    rp = np.asarray(route_pos).reshape(T, K).astype(np.int64)
    order = np.argsort(ids, axis=1, kind="stable")  # ascending expert id
    out = np.zeros((T, y_packed.shape[1]), dtype=f64)
    w = np.asarray(weights, dtype=f64)
    tt = np.arange(T)
    for p in range(K):
        k = order[:, p]
        pos = rp[tt, k]
        live = pos >= 0
        out[live] += w[tt[live], k[live]][:, None] * y_packed[pos[live]]
    if y_shared is not None:
        out += np.asarray(y_shared, dtype=f64)
    if out_prev is not None:
        out += np.asarray(out_prev, dtype=f64)
    return out


def relu2_zero_fraction(h):
    """Fraction of post-ReLU^2 activations that are exactly zero
    ([8 GB Super] "The engine, step by step", item 4).  The pages print it
    only for trained weights; pinned by closed forms on hand-made rows."""
    h = np.asarray(h)
    return float(np.count_nonzero(h == 0)) / max(h.size, 1)


# ---------------------------------------------------------------------------
# The whole layer
# ---------------------------------------------------------------------------

def _front(p, x, w, out_prev):
    """With ``p["prenorm_residual"]`` the input is the hidden state ``H``: the
    layer runs on ``rms_norm(H)`` and ``H`` joins the output sum last as the
    residual ([M6.1] 0x06F.1, ``R_t = H_t + Y_t``)."""
    if not p.get("prenorm_residual"):
        return np.asarray(x, dtype=f64), out_prev
    assert out_prev is None
    h = np.asarray(x, dtype=f64)
    return rms_norm(h, w["w_norm"], p["norm_eps"], p.get("act_dtype", "bf16")), h


def layer_forward(p, x, w, out_prev=None):
    """Expert-major forward of the routed ReLU^2 MoE layer.

    ``p``: dict with d, E, K, F, F_shared, d_latent, n_group, topk_group,
    norm_topk_prob, routed_scaling_factor, and optionally prenorm_residual,
    norm_eps, act_dtype (with w_norm [d] in ``w``; see ``_front``),
    capacity_factor (> 0: the capacity-bounded variant, see
    ``arbitrate_capacity``) and expert_dtype ("fp8": the experts' weights
    quantised by ``quantize_rows_fp8``; "mxfp4": by
    ``quantize_blocks_mxfp4``).  ``w``: dict of float arrays in
    PyTorch storage order: w_router [E, d], bias [E] or None, w_up
    [E, F, d_e], w_down [E, d_e, F], w_up_shared [F_s, d], w_down_shared
    [d, F_s], and for a latent layer w_latent_in [L, d], w_latent_out [d, L].

    Order ([Nemotron circuit] "The Four Layer Kinds CKE Must Preserve": moe =
    router -> group-limited top-k -> routed ReLU2 experts + shared expert):
    router logits on the full-width input, route, dispatch, experts on ``x``
    (or on the latent projection ``x W_lin^T``), combine, and for a latent
    layer one projection back to ``d`` after the combine ([8 GB Super]
    "The only number that matters": experts work in a 1024-wide latent
    space), then the shared expert on the full-width input is added.
    """
    x, out_prev = _front(p, x, w, out_prev)
    w = quantised_expert_weights(w, p.get("expert_dtype"))
    K = p["K"]
    z = router_logits(x, w["w_router"])
    ids, gw, info = route(z, w.get("bias"), p["n_group"], p["topk_group"], K,
                          p["norm_topk_prob"], p["routed_scaling_factor"])
    counts, offsets, route_src, route_pos = dispatch(ids, p["E"])
    cf = p.get("capacity_factor", 0)
    if cf:
        # the capacity-bounded variant: arbitrate, then dispatch only the
        # accepted routes ([M6.1] 0x07 "Minimal Capacity-Aware Pseudocode")
        accept, _ = arbitrate_capacity(ids, gw, capacity_slots(x.shape[0], K, p["E"], cf))
        counts, offsets, route_src, route_pos = dispatch_accepted(ids, accept, p["E"])
    latent = bool(p.get("d_latent", 0))
    x_e = x @ np.asarray(w["w_latent_in"], dtype=f64).T if latent else x
    aq = activation_quantiser(p.get("expert_dtype"), p.get("act_dtype", "bf16"))
    y_packed = run_experts(x_e, route_src, offsets, K, w["w_up"], w["w_down"], aq)
    y_s = None
    if p.get("F_shared", 0):
        y_s = shared_expert(x, w["w_up_shared"], w["w_down_shared"], aq)
    if latent:
        y_lat = combine(y_packed, gw, ids, route_pos)
        out = y_lat @ np.asarray(w["w_latent_out"], dtype=f64).T
        if y_s is not None:
            out = out + y_s
        if out_prev is not None:
            out = out + np.asarray(out_prev, dtype=f64)
    else:
        out = combine(y_packed, gw, ids, route_pos, y_s, out_prev)
    return {"logits": z, "ids": ids, "weights": gw, "route_info": info,
            "counts": counts, "offsets": offsets, "route_src": route_src,
            "route_pos": route_pos, "y_packed": y_packed, "y_shared": y_s,
            "out": out}


def token_major_forward(p, x, w, rows=None, out_prev=None):
    """Token-major schedule: for each row, run its selected experts at once
    ([Nemotron circuit] "Routing Is Cheap; Expert Memory Is The Hard Part":
    the token-major reference, simple and useful for correctness).

    Computes only the listed ``rows`` (all rows by default), one token at a
    time with plain loops, so it also serves as the sampled oracle at full
    size.  Returns ids, weights and out for those rows.
    """
    x, out_prev = _front(p, x, w, out_prev)
    w = quantised_expert_weights(w, p.get("expert_dtype"))
    T = x.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    K = p["K"]
    latent = bool(p.get("d_latent", 0))
    w_r = np.asarray(w["w_router"], dtype=f64)
    aq = activation_quantiser(p.get("expert_dtype"), p.get("act_dtype", "bf16"))
    accept_all = None
    if p.get("capacity_factor", 0):
        # arbitration depends on every row of the routing group
        ids_b, gw_b, _ = route(router_logits(x, w_r), w.get("bias"), p["n_group"], p["topk_group"], K,
                               p["norm_topk_prob"], p["routed_scaling_factor"])
        accept_all, _ = arbitrate_capacity(ids_b, gw_b, capacity_slots(T, K, p["E"], p["capacity_factor"]))
    out = np.zeros((len(rows), x.shape[1]), dtype=f64)
    ids_all = np.zeros((len(rows), K), dtype=np.int32)
    w_all = np.zeros((len(rows), K), dtype=f64)
    for i, t in enumerate(rows):
        xt = x[t]
        z = np.array([[float(np.dot(xt, w_r[e])) for e in range(w_r.shape[0])]])
        ids, gw, _ = route(z, w.get("bias"), p["n_group"], p["topk_group"], K,
                           p["norm_topk_prob"], p["routed_scaling_factor"])
        ids_all[i], w_all[i] = ids[0], gw[0]
        xe = xt @ np.asarray(w["w_latent_in"], dtype=f64).T if latent else xt
        acc = np.zeros(xe.shape[0], dtype=f64)
        for k in np.argsort(ids[0], kind="stable"):
            if accept_all is not None and not accept_all[t, k]:
                continue
            e = int(ids[0, k])
            acc += gw[0, k] * expert_mlp(xe[None, :], w["w_up"][e], w["w_down"][e], aq)[0]
        if latent:
            acc = acc @ np.asarray(w["w_latent_out"], dtype=f64).T
        if p.get("F_shared", 0):
            acc += shared_expert(xt[None, :], w["w_up_shared"], w["w_down_shared"], aq)[0]
        if out_prev is not None:
            acc += np.asarray(out_prev[t], dtype=f64)
        out[i] = acc
    return {"ids": ids_all, "weights": w_all, "out": out}


def row_relative_error(y, y_ref):
    """Max over rows of ``||y_t - yref_t||_2 / ||yref_t||_2`` and the global
    ``max|y - yref| / max|yref|`` (the two error measures reported).  Rows
    whose reference norm is zero compare absolutely."""
    y = np.asarray(y, dtype=f64)
    y_ref = np.asarray(y_ref, dtype=f64)
    num = np.linalg.norm(y - y_ref, axis=1)
    den = np.linalg.norm(y_ref, axis=1)
    rel = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    glob = float(np.max(np.abs(y - y_ref)) / max(np.max(np.abs(y_ref)), 1e-300))
    return float(rel.max() if rel.size else 0.0), glob


# ---------------------------------------------------------------------------
# Backward pass (gradients of a loss L through the layer output Y)
# ---------------------------------------------------------------------------
#
# [M6.1] 0x06F derives the single-device backward of a routed MoE layer for
# a softmax router and SwiGLU experts: the combine adjoint is a broadcast and
# a dot product (0x06F.2), the selected gates' Jacobian couples the K routes
# of a token (0x06F.3), the router projection returns G_Z^T H and G_Z W_r
# (0x06F.4), the expert's own backward (0x06F.5) and the gather adjoint as a
# scatter-add (0x06F.6).  [Nemotron circuit] "Nemotron is not one circuit"
# announces the same derivation for this layer.  Here the same steps are
# taken for the sigmoid router with normalised selected weights and the
# ReLU^2 expert.  The selected ids are saved metadata (no gradient); the
# correction bias only chooses experts and receives none.  ``dY`` is the
# gradient of the loss with respect to the layer output Y (the residual of
# ``R = H + Y`` is outside the operator: the caller adds dY to dH for it).


def gate_backward(s_sel, q, norm_topk_prob, routed_scaling_factor):
    """Gradient of the loss with respect to the selected router logits.

    ``s_sel`` [T, K]: the selected experts' sigmoid scores; ``q`` [T, K]:
    the loss gradient with respect to each gate weight g (0x06F.2:
    ``q = <dY_t, U_{t,k}>`` for an accepted route, 0 for a dropped one).
    With ``g_k = rsf * s_k / S``, ``S = sum_j s_j`` (normalised), the
    Jacobian ``dg_j / ds_k = (rsf [j = k] - g_j) / S`` gives
    ``dL/ds_k = (rsf q_k - sum_j g_j q_j) / S``; without normalisation
    ``dL/ds_k = rsf q_k``.  Then ``dL/dz_k = dL/ds_k * s_k (1 - s_k)`` (the
    sigmoid's derivative).  A dropped route (q = 0) still receives
    ``-s(1-s) sum_j g_j q_j / S``: it takes part in the normaliser (the
    same coupling 0x06F.3 points out for the selected softmax)."""
    s_sel = np.asarray(s_sel, dtype=f64)
    q = np.asarray(q, dtype=f64)
    rsf = float(routed_scaling_factor)
    if norm_topk_prob:
        S = s_sel.sum(axis=1, keepdims=True)
        g = rsf * s_sel / S
        ds = (rsf * q - (g * q).sum(axis=1, keepdims=True)) / S
    else:
        ds = rsf * q
    return ds * s_sel * (1.0 - s_sel)


def expert_backward(x_rows, w_up_e, w_down_e, dU):
    """Backward of one ReLU^2 expert ``U = W_down relu(W_up x)^2`` over its
    rows (the ReLU^2 counterpart of [M6.1] 0x06F.5): with ``u = W_up x``,
    ``a = relu(u)``, ``h = a^2``: ``dh = dU W_down`` (rows), ``du = dh * 2a``
    (ReLU^2' = 2 relu), ``dW_down = dU^T h``, ``dW_up = du^T x``,
    ``dx = du W_up``.  Parameter gradients sum over the expert's rows."""
    x_rows = np.asarray(x_rows, dtype=f64)
    w_up_e = np.asarray(w_up_e, dtype=f64)
    w_down_e = np.asarray(w_down_e, dtype=f64)
    dU = np.asarray(dU, dtype=f64)
    u = x_rows @ w_up_e.T
    a = np.maximum(u, 0.0)
    h = a * a
    dh = dU @ w_down_e
    du = dh * 2.0 * a
    return {"dx": du @ w_up_e, "dw_up": du.T @ x_rows, "dw_down": dU.T @ h}


def gather_adjoint(dx, toks, dx_rows):
    """The adjoint of the dispatch gather ([M6.1] 0x06F.6): each packed
    row's input gradient is added to its token's row, never written over (a
    token with several routes owns several rows)."""
    for i, t in enumerate(toks):
        dx[t] += dx_rows[i]
    return dx


def layer_backward(p, x, w, dY):
    """Gradients of ``L`` (with ``dL/dY = dY`` [T, d]) with respect to the
    layer input ``x`` and every weight, following [M6.1] 0x06F's steps:

    1. the forward relation is frozen: ids, gates, admissions and route maps
       of ``layer_forward``;
    2. combine adjoint (0x06F.2): ``dU_r = A_r g_r dY_t`` and
       ``q_r = A_r <dY_t, U_r>`` per route r = (t, k), A_r the admission;
    3. gate adjoint (``gate_backward``) into the selected logits ``G_Z``
       (zero elsewhere; the bias gets none);
    4. router projection (0x06F.4): ``dW_r = G_Z^T x``, ``dx += G_Z W_r``;
    5. each expert's backward over its accepted rows (``expert_backward``),
       the shared expert's with ``dU = dY`` (weight 1);
    6. gather adjoint (0x06F.6): each route's ``dx`` row is added (never
       written over) to its token's row.

    With the fused front and back (``p["prenorm_residual"]``: the input is
    the hidden state ``H``, the layer runs on ``x = rms_norm(H)`` and ``out =
    Y + H``), the steps above run on ``x`` and then ``dH = dY + J^T dx``
    through the norm (``rms_norm_backward``; the one rounding of ``x`` to the
    activation dtype is taken as the identity, its derivative being zero
    almost everywhere), and ``dw_norm`` is returned too.

    A latent layer (``p["d_latent"]`` = L; ``layer_forward``'s order: the
    router and the shared expert on ``x``, the routed experts on ``x_lat =
    x W_lin^T``, their combine ``y_lat`` [T, L] projected back by ``out =
    y_lat W_lout^T + y_s``) differentiates the two projections as the linear
    maps they are: ``dy_lat = dY W_lout`` and ``dW_lout = dY^T y_lat``; the
    combine and gate adjoints use ``dy_lat`` and the latent ``U``; the
    router's and the shared expert's gradients are taken on ``x`` as above;
    the experts' input gradients, gathered per token into ``dx_lat`` [T, L],
    reach ``x`` through ``dx += dx_lat W_lin``, and ``dW_lin = dx_lat^T x``.

    Scope: dropless or capacity-bounded.  Returns dx [T, d], dw_router [E,
    d], dw_up [E, F, d_e], dw_down [E, d_e, F] (d_e = L for a latent layer,
    else d), dw_up_shared, dw_down_shared (None without a shared expert),
    dw_norm (None without the fused front), dw_latent_in [L, d] and
    dw_latent_out [d, L] (None without latent projections), and the
    per-route ``q`` and ``dz`` [T, K]."""
    if p.get("prenorm_residual"):
        h = np.asarray(x, dtype=f64)
        xn = rms_norm(h, w["w_norm"], p["norm_eps"], p.get("act_dtype", "bf16"))
        g = layer_backward(dict(p, prenorm_residual=0), xn, w, dY)
        dh, dw_norm = rms_norm_backward(h, w["w_norm"], p["norm_eps"], g["dx"])
        g["dx"] = np.asarray(dY, dtype=f64) + dh
        g["dw_norm"] = dw_norm
        return g
    w = quantised_expert_weights(w, p.get("expert_dtype"))
    fw = layer_forward(p, x, w)
    x = np.asarray(x, dtype=f64)
    dY = np.asarray(dY, dtype=f64)
    T, d = x.shape
    K, E = p["K"], p["E"]
    ids, g = fw["ids"], fw["weights"]
    rp = np.asarray(fw["route_pos"]).reshape(T, K).astype(np.int64)
    U = fw["y_packed"]
    latent = bool(p.get("d_latent", 0))
    if latent:
        # the projections around the latent experts
        w_lin = np.asarray(w["w_latent_in"], dtype=f64)    # [L, d]
        w_lout = np.asarray(w["w_latent_out"], dtype=f64)  # [d, L]
        x_e = x @ w_lin.T
        y_lat = combine(U, g, ids, fw["route_pos"])
        dY_e = dY @ w_lout
        dw_latent_out = dY.T @ y_lat
    else:
        x_e, dY_e = x, dY
    de = x_e.shape[1]
    # 2. combine adjoint
    q = np.zeros((T, K), dtype=f64)
    R = len(U)
    dU = np.zeros((R, de), dtype=f64)
    for t in range(T):
        for k in range(K):
            r = rp[t, k]
            if r < 0:
                continue
            q[t, k] = float(dY_e[t] @ U[r])
            dU[r] = g[t, k] * dY_e[t]
    # 3. gate adjoint
    s = sigmoid(fw["logits"])
    s_sel = np.take_along_axis(s, ids.astype(np.int64), axis=1)
    dz = gate_backward(s_sel, q, p["norm_topk_prob"], p["routed_scaling_factor"])
    GZ = np.zeros((T, E), dtype=f64)
    for t in range(T):
        for k in range(K):
            GZ[t, ids[t, k]] += dz[t, k]
    # 4. router projection
    w_r = np.asarray(w["w_router"], dtype=f64)
    dw_router = GZ.T @ x
    dx = GZ @ w_r
    # 5. experts over their accepted rows, 6. gather adjoint (into the
    # experts' input: x, or x_lat for a latent layer)
    F = np.asarray(w["w_up"][0]).shape[0]
    dw_up = np.zeros((E, F, de), dtype=f64)
    dw_down = np.zeros((E, de, F), dtype=f64)
    dx_e = np.zeros((T, de), dtype=f64)
    offsets, route_src = fw["offsets"], fw["route_src"]
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        toks = np.asarray(route_src[a:b]) // K
        gb = expert_backward(x_e[toks], w["w_up"][e], w["w_down"][e], dU[a:b])
        dw_up[e] = gb["dw_up"]
        dw_down[e] = gb["dw_down"]
        gather_adjoint(dx_e, toks, gb["dx"])
    dw_latent_in = None
    if latent:
        dx += dx_e @ w_lin
        dw_latent_in = dx_e.T @ x
    else:
        dw_latent_out = None
        dx += dx_e
    dw_up_s = dw_down_s = None
    if p.get("F_shared", 0):
        gs = expert_backward(x, w["w_up_shared"], w["w_down_shared"], dY)
        dx += gs["dx"]
        dw_up_s, dw_down_s = gs["dw_up"], gs["dw_down"]
    return {"dx": dx, "dw_router": dw_router, "dw_up": dw_up, "dw_down": dw_down,
            "dw_up_shared": dw_up_s, "dw_down_shared": dw_down_s, "dw_norm": None,
            "dw_latent_in": dw_latent_in, "dw_latent_out": dw_latent_out, "q": q, "dz": dz,
            "forward": fw}
