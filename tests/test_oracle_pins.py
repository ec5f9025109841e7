"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each ``check_*`` function raises AssertionError on a mismatch.  The tests
call them on the oracle as written; ``test_mutations_are_caught`` plants one
plausible mistake at a time in the oracle (on the CPU, by patching one of
its functions) and requires that at least one pin fails, so a pin that
cannot tell a right oracle from a wrong one is itself caught.

Sources (page title and section):
* "Nemotron is not one circuit" -- "The Router Is A Deterministic
  Algorithm", "The C Kernel Contract".
* "M6.1 - Routed Capacity" -- 0x05A (route table), 0x05C (P^T P = diag(k)),
  0x05D (combine trace), 0x05F (residual outside, add not overwrite),
  0x06C.2 (token-choice table).
* "NemotronH" -- "Arithmetic" (fp32 router, bias for the choice only, ties
  to the lower id, ascending-id combine; RMS norm in fp32 times the plain
  weight).
* "M6.1 - Routed Capacity" -- 0x06F.1 (the residual ``R_t = H_t + Y_t``
  outside the MoE operator); 0x06 and 0x06A (capacity ``C = ceil(CF T k /
  E)``, its worked numbers, per-group arbitration, the focal-token example,
  the arbitration order), 0x07 (the sequential capacity-aware sketch, which
  accepts the same routes), 0x05F (fixed drop: no renormalisation).
* The OCP 8-bit floating point format E4M3 (published specification): the
  field layout and the values it names (448 the largest, 2^-6 the smallest
  normal, 2^-9 the smallest subnormal, S.1111.111 the NaN).
"""
import contextlib
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle.moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# brute force router on tiny inputs, in exact rational arithmetic
# ---------------------------------------------------------------------------

def brute_select(c_row, n_group, topk_group, K):
    """Enumerate every group subset and every expert subset.

    Group score = the largest sum of two distinct members (the sum of the
    two largest).  The kept groups are the ``topk_group``-subset with the
    largest total score, ties to the lexicographically smallest index tuple;
    the chosen experts are the ``K``-subset of eligible experts with the
    largest total corrected score, ties likewise.  Returned in descending
    score, equal scores in ascending id.
    """
    E = len(c_row)
    c = [Fraction(float(v)) for v in c_row]
    gs = E // n_group
    if n_group > 1:
        G = [max(c[a] + c[b] for a, b in itertools.combinations(range(g * gs, (g + 1) * gs), 2))
             for g in range(n_group)]
        best, best_set = None, None
        for sub in itertools.combinations(range(n_group), topk_group):
            s = sum(G[g] for g in sub)
            if best is None or s > best:
                best, best_set = s, sub
        eligible = [e for g in best_set for e in range(g * gs, (g + 1) * gs)]
    else:
        eligible = list(range(E))
    best, best_set = None, None
    for sub in itertools.combinations(sorted(eligible), K):
        s = sum(c[e] for e in sub)
        if best is None or s > best:
            best, best_set = s, sub
    return sorted(best_set, key=lambda e: (-c[e], e))


def check_selection_brute_force(seed=0, n_cases=400):
    rng = np.random.default_rng(seed)
    for case in range(n_cases):
        E = int(rng.choice([4, 8, 12, 16]))
        groups = [g for g in (1, 2, 4) if E % g == 0 and (g == 1 or E // g >= 2)]
        n_group = int(rng.choice(groups))
        topk_group = int(rng.integers(1, n_group + 1))
        max_k = topk_group * (E // n_group)
        K = int(rng.integers(1, min(max_k, 6) + 1))
        # dyadic scores on a coarse grid: fp32 sums are exact and ties frequent
        c = (np.round(rng.uniform(-1, 1, size=(1, E)) * 16) / 16).astype(np.float32)
        elig = O.eligible_experts(c, n_group, topk_group)
        ids = O.select_experts(c, elig, K)[0].tolist()
        want = brute_select(c[0], n_group, topk_group, K)
        assert ids == want, (case, c.tolist(), n_group, topk_group, K, ids, want)


def check_sigmoid_closed_forms():
    z = np.array([0.0, math.log(3.0), -math.log(3.0), math.log(7.0), 40.0, -40.0])
    s = O.sigmoid(z)
    want = np.array([0.5, 0.75, 0.25, 0.875, 1.0 / (1.0 + math.exp(-40.0)), math.exp(-40.0) / (1 + math.exp(-40.0))])
    assert np.allclose(s, want, rtol=1e-15, atol=0.0), (s, want)
    zz = np.linspace(-8, 8, 101)
    assert np.allclose(O.sigmoid(zz) + O.sigmoid(-zz), 1.0, atol=1e-15)


def check_decision_scores():
    # bias is additive on the selection score only; s untouched by the bias
    z = np.array([[0.0, math.log(3.0), -math.log(3.0)]])
    b = np.array([0.25, -0.25, 0.5], dtype=np.float32)
    s64, s32, c32, c64 = O.decision_scores(z, b)
    assert np.array_equal(c32, np.array([[0.75, 0.5, 0.75]], dtype=np.float32)), c32
    assert np.allclose(s64, [[0.5, 0.75, 0.25]], rtol=1e-15)
    assert c32.dtype == np.float32 and s32.dtype == np.float32


def check_router_orientation():
    # W_r stored [E, d]: z[t, e] = sum_j x[t, j] W_r[e, j]
    x = np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]])
    W = np.array([[0, 0, 1], [1, 0, 0], [0, 1, 0], [1, 1, 1]], dtype=np.float32)
    z = O.router_logits(x, W)
    assert np.array_equal(z, [[3, 1, 2, 6], [6, 4, 5, 15]]), z


def check_token_choice_table():
    g = _load("m61_token_choice_top2.json")
    z = np.array(g["affinity"], dtype=np.float64)
    ids, w, info = O.route(z, None, 1, 1, g["K"], 1, 1.0)
    assert ids.tolist() == g["top2"], ids.tolist()
    counts, offsets, _, _ = O.dispatch(ids, 4)
    assert counts.tolist() == g["routes_per_expert"], counts
    assert offsets.tolist() == [0, 6, 11, 14, 16] and offsets[-1] == g["routes_total"]
    assert info["exact_tie"][7] and not info["exact_tie"][:7].any()


def check_group_score_is_top2_sum():
    # group 0 has the single largest expert, group 1 the larger top-2 sum:
    # ranking groups by their maximum would keep group 0.
    c = np.array([[0.9, 0.1, 0.0, 0.0, 0.6, 0.55, 0.0, 0.0]], dtype=np.float32)
    elig = O.eligible_experts(c, 2, 1)
    assert elig[0].tolist() == [False] * 4 + [True] * 4, elig
    ids = O.select_experts(c, elig, 2)
    assert ids.tolist() == [[4, 5]], ids


def check_masked_groups_never_selected():
    # every corrected score negative: a mask value of 0 (instead of
    # "never selectable") would pull masked experts back in
    c = np.array([[-0.1, -0.9, -0.9, -0.9, -0.3, -0.2, -0.9, -0.9]], dtype=np.float32)
    elig = O.eligible_experts(c, 2, 1)  # group 1: -0.5 > group 0: -1.0
    ids = O.select_experts(c, elig, 3)
    assert ids.tolist() == [[5, 4, 6]], ids


def check_tie_rules():
    c = np.array([[0.5, 0.7, 0.5, 0.7, 0.5, 0.1, 0.1, 0.1]], dtype=np.float32)
    ids = O.select_experts(c, np.ones_like(c, dtype=bool), 4)
    assert ids.tolist() == [[1, 3, 0, 2]], ids
    # equal group scores: the lower group index survives
    c2 = np.array([[0.2, 0.3, 0.3, 0.2, 0.0, 0.0]], dtype=np.float32)
    elig = O.eligible_experts(c2, 3, 1)
    assert elig[0].tolist() == [True, True, False, False, False, False], elig


def check_decision_in_fp32():
    # two logits whose sigmoids differ in float64 but round to the same fp32
    # value: the router sees a tie and keeps the lower id, although the
    # higher id has the (slightly) larger float64 score
    z = np.array([[2.0, 2.0 + 1e-9, -3.0]])
    s64, s32, c32, c64 = O.decision_scores(z, None)
    assert s64[0, 1] > s64[0, 0] and s32[0, 1] == s32[0, 0]
    ids, _, info = O.route(z, None, 1, 1, 1, 1, 1.0)
    assert ids.tolist() == [[0]], ids
    assert info["gap"][0] > 0  # the fp64 gap is nonzero: a near-tie, not an exact one


def _logit(pr):
    pr = np.asarray(pr, dtype=np.float64)
    return np.log(pr / (1.0 - pr))


def check_boundary_gap_closed_forms():
    """The near-tie gap in closed form on hand-made rows whose sigmoid
    scores are known: the K-th minus the (K+1)-th eligible corrected score,
    the bias inside the corrected score, and the topk_group-th minus the
    next group score (a group's score is its top-two sum), whichever is
    smaller.  The gap decides which rows the GPU parity tests exempt from
    exact ids, so a gap off by any factor must fail here."""
    def gap(s, bias, ng, tg, K):
        z = _logit(np.array([s]))
        b = None if bias is None else np.array(bias, dtype=np.float32)
        return O.route(z, b, ng, tg, K, 1, 1.0)[2]["gap"][0]

    s = [0.9, 0.8, 0.7, 0.6, 0.5, 0.4]
    assert abs(gap(s, None, 1, 1, 2) - 0.1) < 1e-12
    assert abs(gap(s, None, 1, 1, 4) - 0.1) < 1e-12
    # the bias moves expert 2 between experts 0 and 1: c = .9, .8, .85(+.15)
    bias = [0.0, 0.0, 0.15, 0.0, 0.0, 0.0]
    b32 = float(np.float32(0.15))
    assert abs(gap(s, bias, 1, 1, 2) - (0.7 + b32 - 0.8)) < 1e-12
    # K = E: nothing is left out, no expert boundary
    assert gap(s, None, 1, 1, 6) == math.inf
    # groups of two: G = 1.7, 1.3, 0.9; one group kept holds exactly K = 2
    # experts, so only the group boundary counts: 1.7 - 1.3
    assert abs(gap(s, None, 3, 1, 2) - 0.4) < 1e-12
    # two groups kept: expert boundary .8 - .7 = .1 beats the group one (.4)
    assert abs(gap(s, None, 3, 2, 2) - 0.1) < 1e-12
    # the group boundary is the smaller one: G = 1.1, 1.15, 0.95
    s2 = [0.9, 0.2, 0.85, 0.3, 0.5, 0.45]
    assert abs(gap(s2, None, 3, 1, 1) - 0.05) < 1e-12
    # kept groups 1, 0 (1.15, 1.1): experts .9 .85 .3 .2; K = 1 -> .9 - .85
    assert abs(gap(s2, None, 3, 2, 1) - 0.05) < 1e-12
    assert abs(gap(s2, None, 3, 2, 3) - min(0.3 - 0.2, 1.1 - 0.95)) < 1e-12


def check_weights(seed=1):
    rng = np.random.default_rng(seed)
    T, E, K = 50, 16, 4
    z = rng.normal(size=(T, E))
    b = rng.normal(scale=0.3, size=E).astype(np.float32)
    for rsf in (1.0, 2.5):
        ids, w, _ = O.route(z, b, 4, 2, K, 1, rsf)
        s = O.sigmoid(z)
        sel = np.take_along_axis(s, ids.astype(np.int64), axis=1)
        assert np.allclose(w.sum(axis=1), rsf, rtol=0, atol=1e-12 * rsf), w.sum(axis=1)
        assert np.allclose(w, rsf * sel / sel.sum(axis=1, keepdims=True), rtol=1e-14)
        ids2, w2, _ = O.route(z, b, 4, 2, K, 0, rsf)
        assert np.array_equal(ids, ids2)
        assert np.allclose(w2, rsf * sel, rtol=1e-14)
        # selection respects the corrected score: every selected eligible
        # score >= every unselected eligible score
        _, _, c32, _ = O.decision_scores(z, b)
        elig = O.eligible_experts(c32, 4, 2)
        for t in range(T):
            chosen = set(ids[t].tolist())
            lo = min(c32[t, e] for e in chosen)
            rest = [c32[t, e] for e in range(E) if elig[t, e] and e not in chosen]
            assert not rest or lo >= max(rest)
            assert len(chosen) == K


def check_dispatch_fixture():
    g = _load("m61_dispatch_route_table.json")
    ids = np.array(g["expert_of_route"], dtype=np.int32)
    counts, offsets, route_src, route_pos = O.dispatch(ids, g["E"])
    assert route_src.tolist() == g["packed_route_ids"], route_src
    assert offsets.tolist() == g["offsets"], offsets
    K = g["K"]
    assert (route_src // K).tolist() == g["packed_tokens"]
    ex = ids.reshape(-1)[route_src]
    assert ex.tolist() == g["packed_experts"]
    local = [j - offsets[e] for j, e in enumerate(ex)]
    assert local == g["expert_local_rows"]


def check_dispatch_round_trip(seed=2):
    rng = np.random.default_rng(seed)
    for _ in range(20):
        T, E = int(rng.integers(1, 40)), int(rng.integers(2, 20))
        K = int(rng.integers(1, E + 1))
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
        counts, offsets, route_src, route_pos = O.dispatch(ids, E)
        R = T * K
        assert np.array_equal(route_src[route_pos], np.arange(R))
        assert np.array_equal(route_pos[route_src], np.arange(R))
        assert offsets[0] == 0 and offsets[-1] == R and np.array_equal(np.diff(offsets), counts)
        assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E))
        # packed rows are expert-contiguous and in (token, slot) order inside
        ex = ids.reshape(-1)[route_src]
        for e in range(E):
            seg = route_src[offsets[e]:offsets[e + 1]]
            assert np.all(ex[offsets[e]:offsets[e + 1]] == e)
            assert np.all(np.diff(seg) > 0)
        # gather by route_src, scatter back by route_pos: every (t, k) sees x[t]
        x = rng.normal(size=(T, 3))
        packed = x[route_src // K]
        back = packed[route_pos].reshape(T, K, 3)
        assert np.array_equal(back, np.repeat(x[:, None, :], K, axis=1))
        # identity experts, unit weights: P^T P = diag(K) gives K * x
        y = O.combine(packed, np.ones((T, K)), ids, route_pos)
        assert np.allclose(y, K * x, rtol=1e-15, atol=0)


def check_combine_trace():
    g = _load("m61_combine_trace.json")
    H = np.array(g["H"], dtype=np.float64)
    ids = np.array(g["expert_of_route"], dtype=np.int32)
    gates = np.array(g["gate_of_route"], dtype=np.float64)
    ex = g["experts"]

    def expert(e, v):
        p = ex["E%d" % e]
        return p["scale"] * v + np.array(p["shift"])

    counts, offsets, route_src, route_pos = O.dispatch(ids, 3)
    K = ids.shape[1]
    y_packed = np.stack([expert(ids.reshape(-1)[r], H[r // K]) for r in route_src])
    Y = O.combine(y_packed, gates, ids, route_pos)
    assert np.allclose(Y, np.array(g["Y"]), rtol=0, atol=1e-12), Y


def _random_layer(rng, T, d, E, K, F, Fs, n_group=1, topk_group=1, rsf=1.5, latent=0):
    de = latent or d
    p = {"d": d, "E": E, "K": K, "F": F, "F_shared": Fs, "d_latent": latent,
         "n_group": n_group, "topk_group": topk_group, "norm_topk_prob": 1,
         "routed_scaling_factor": rsf}
    w = {"w_router": rng.normal(scale=0.3, size=(E, d)).astype(np.float32),
         "bias": rng.normal(scale=0.05, size=E).astype(np.float32),
         "w_up": rng.normal(scale=d ** -0.5, size=(E, F, de)),
         "w_down": rng.normal(scale=F ** -0.5, size=(E, de, F))}
    if Fs:
        w["w_up_shared"] = rng.normal(scale=d ** -0.5, size=(Fs, d))
        w["w_down_shared"] = rng.normal(scale=Fs ** -0.5, size=(d, Fs))
    x = rng.normal(size=(T, d))
    return p, w, x


def check_dense_equivalent(seed=3):
    """K = E, one group, zero router: every weight is rsf/E and the layer is
    the textbook dense ReLU^2 MLP over the concatenated experts."""
    rng = np.random.default_rng(seed)
    T, d, E, F, Fs, rsf = 9, 12, 5, 7, 6, 2.5
    p, w, x = _random_layer(rng, T, d, E, E, F, Fs, rsf=rsf)
    w["w_router"] = np.zeros((E, d), dtype=np.float32)
    w["bias"] = rng.normal(scale=0.2, size=E).astype(np.float32)  # bias must not reach the weights
    r = O.layer_forward(p, x, w)
    assert np.allclose(r["weights"], rsf / E, rtol=1e-15)
    up_cat = np.concatenate(list(w["w_up"]), axis=0)            # [E*F, d]
    down_cat = np.concatenate(list(w["w_down"]), axis=1)        # [d, E*F]
    hid = np.maximum(x @ up_cat.T, 0.0) ** 2
    dense = (rsf / E) * hid @ down_cat.T
    dense += (np.maximum(x @ w["w_up_shared"].T, 0.0) ** 2) @ w["w_down_shared"].T
    err = np.max(np.abs(r["out"] - dense)) / np.max(np.abs(dense))
    assert err < 1e-12, err
    assert r["ids"].tolist() == [sorted(range(E), key=lambda e: (-float(0.5 + w["bias"][e]), e))] * T


def check_token_major_matches_expert_major(seed=4):
    rng = np.random.default_rng(seed)
    for (n_group, topk_group) in ((1, 1), (4, 2)):
        p, w, x = _random_layer(rng, 24, 32, 8, 3, 16, 12, n_group, topk_group)
        a = O.layer_forward(p, x, w)
        b = O.token_major_forward(p, x, w)
        assert np.array_equal(a["ids"], b["ids"])
        err = np.max(np.abs(a["out"] - b["out"])) / np.max(np.abs(a["out"]))
        assert err < 1e-13, err


def check_latent_scaling(seed=5):
    """Latent layer with W_lin = 2 I and W_lout = I / 4 equals the plain
    layer: ReLU^2 is homogeneous of degree 2, so the experts return 4x on 2x
    inputs.  The router must read the full-width x (reading it from the
    latent projection doubles the logits and changes the choice)."""
    rng = np.random.default_rng(seed)
    d = 16
    p, w, x = _random_layer(rng, 20, d, 8, 2, 10, 6, latent=d)
    w["w_router"] = (w["w_router"] * 4).astype(np.float32)
    w["w_latent_in"] = 2.0 * np.eye(d)
    w["w_latent_out"] = 0.25 * np.eye(d)
    lat = O.layer_forward(p, x, w)
    p2 = dict(p, d_latent=0)
    plain = O.layer_forward(p2, x, w)
    assert np.array_equal(lat["ids"], plain["ids"])
    assert np.allclose(lat["out"], plain["out"], rtol=1e-13, atol=1e-13)


def check_latent_orientation(seed=51):
    """A latent layer with a non-symmetric permutation P: W_lin = 2 P,
    W_lout = P^T / 4 and every expert conjugated by P (up W P^T, down P W)
    equals the plain layer (the experts see P(2x), return 4 P y, and P^T / 4
    maps it back).  A projection applied transposed (P^T instead of P)
    scrambles the latent coordinates and fails."""
    rng = np.random.default_rng(seed)
    d = 12
    p, w, x = _random_layer(rng, 16, d, 6, 2, 10, 6, latent=d)
    P = np.roll(np.eye(d), 1, axis=0)          # cyclic shift: P != P^T
    P[[0, 5]] = P[[5, 0]]
    assert not np.allclose(P, P.T)
    plain = O.layer_forward(dict(p, d_latent=0), x, w)
    wl = dict(w)
    wl["w_latent_in"] = 2.0 * P
    wl["w_latent_out"] = 0.25 * P.T
    wl["w_up"] = np.stack([u @ P.T for u in w["w_up"]])
    wl["w_down"] = np.stack([P @ dn for dn in w["w_down"]])
    lat = O.layer_forward(p, x, wl)
    assert np.array_equal(lat["ids"], plain["ids"])
    assert np.allclose(lat["out"], plain["out"], rtol=1e-12, atol=1e-12)
    tm = O.token_major_forward(p, x, wl)
    assert np.allclose(tm["out"], plain["out"], rtol=1e-12, atol=1e-12)


def check_relu2_zero_fraction():
    """Exact zeros after ReLU^2, closed form: negative, zero and negative-zero
    pre-activations give 0, positive ones do not; an input aligned with
    alternating-sign rows zeroes exactly half the neurons."""
    h = O.relu2(np.array([[-1.5, 0.0, -0.0, 2.0], [0.25, -3.0, 1.0, 4.0]]))
    assert O.relu2_zero_fraction(h) == 4 / 8
    assert O.relu2_zero_fraction(np.zeros((3, 5))) == 1.0
    assert O.relu2_zero_fraction(np.ones((3, 5))) == 0.0
    F, d = 10, 6
    w_up = np.zeros((F, d))
    w_up[:, 0] = [(-1.0) ** f * (f + 1) for f in range(F)]
    x = np.zeros((1, d))
    x[0, 0] = 0.5
    assert O.relu2_zero_fraction(O.relu2(x @ w_up.T)) == 0.5
    assert O.relu2_zero_fraction(O.relu2(-x @ w_up.T)) == 0.5
    x[0, 0] = 0.0
    assert O.relu2_zero_fraction(O.relu2(x @ w_up.T)) == 1.0


def check_accumulate_out(seed=6):
    rng = np.random.default_rng(seed)
    p, w, x = _random_layer(rng, 10, 16, 4, 2, 8, 8)
    prev = rng.normal(size=(10, 16))
    a = O.layer_forward(p, x, w)["out"]
    b = O.layer_forward(p, x, w, out_prev=prev)["out"]
    assert np.allclose(b - a, prev, rtol=0, atol=1e-13)


def check_relu2():
    assert O.relu2(np.array([-1.5, -0.0, 0.0, 2.0, 3.5])).tolist() == [0.0, 0.0, 0.0, 4.0, 12.25]


# ---------------------------------------------------------------------------
# RMSNorm in front of the layer, residual behind it
# ---------------------------------------------------------------------------

def _bf16_near(a, b, max_ulps=1):
    """a, b: float64 arrays of bf16 values; |a - b| within max_ulps bf16 ulps."""
    a, b = np.asarray(a), np.asarray(b)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(b), 1e-30))) - 7)
    return bool(np.all(np.abs(a - b) <= max_ulps * ulp))


def check_rms_norm_worked_example():
    # 1..8: mean of squares 204 / 8 = 25.5, so y_i = i / sqrt(25.5) * w_i
    h = np.arange(1, 9, dtype=np.float64)[None, :]
    w = np.array([1.0, 0.5, 2.0, -1.0, 1.0, 1.0, 0.25, 3.0])
    y = O.rms_norm(h, w, 0.0, "f32")[0]
    exact = np.arange(1, 9) / math.sqrt(25.5) * w
    assert np.allclose(y, exact, rtol=3e-7, atol=0)
    yb = O.rms_norm(h, w, 0.0, "bf16")[0]
    assert _bf16_near(yb, O.round_to_act(exact, "bf16"))


def check_rms_norm_constant_row():
    # a constant row c has rms |c|: with eps = 0 the result is sign(c) * w
    d = 64
    w = np.linspace(-2.0, 2.0, d)
    w32 = w.astype(np.float32).astype(np.float64)
    for c in (0.75, -3.0, 1.0):
        y = O.rms_norm(np.full((1, d), c), w, 0.0, "f32")[0]
        assert np.array_equal(y, np.sign(c) * w32), c
    # eps is added to the mean of squares: c = 1, eps = 3 gives 1 / 2
    y = O.rms_norm(np.ones((1, d)), np.ones(d), 3.0, "f32")[0]
    assert np.all(y == 0.5)


def check_rms_norm_rounds_once():
    """The norm is the exact value rounded once to the activation dtype.
    A constant row c has rms |c|, so with eps = 0 the exact result is w
    itself; weights a hair above a bfloat16 midpoint must round up, which a
    detour through fp32 (rounding onto the midpoint, then to even) gets
    wrong."""
    d = 8
    mid = 1.0 + 2.0 ** -8                       # midpoint of 1 and 1 + 2^-7
    w = np.array([mid + 2.0 ** -30, mid, 1.0 + 3 * 2.0 ** -8, mid - 2.0 ** -30,
                  -(mid + 2.0 ** -30), 2.0, 0.5, 1.0])
    yb = O.rms_norm(np.full((1, d), 2.5), w, 0.0, "bf16")[0]
    want = [1.0 + 2.0 ** -7, 1.0, 1.0 + 2.0 ** -6, 1.0, -(1.0 + 2.0 ** -7), 2.0, 0.5, 1.0]
    assert yb.tolist() == want, yb
    # fp32 activations: the exact value rounded to fp32 once
    y32 = O.rms_norm(np.full((1, d), -4.0), w, 0.0, "f32")[0]
    assert y32.tolist() == (-w).astype(np.float32).astype(np.float64).tolist()
    # scaling a row by a power of two changes nothing when eps = 0
    rng = np.random.default_rng(8)
    h = O.round_to_act(rng.normal(size=(6, 264)) * 3.0, "bf16")
    wn = O.round_to_act(1.0 + 0.1 * rng.normal(size=264), "bf16")
    assert np.array_equal(O.rms_norm(4.0 * h, wn, 0.0, "bf16"), O.rms_norm(h, wn, 0.0, "bf16"))


def check_round_once():
    """float64 -> bfloat16 in one rounding, ties to even: the named cases,
    the subnormal spacing 2^-133, and agreement with the bit-level fp32 ->
    bfloat16 rounding on values that are already fp32."""
    one = 1.0
    vals = [one, one + 2.0 ** -8, one + 3 * 2.0 ** -8, one + 2.0 ** -8 + 2.0 ** -40, -2.5, 0.0,
            2.0 ** -130 + 2.0 ** -134, 3 * 2.0 ** -134, 3.0e38 * 1.2]
    got = O.round_once(np.array(vals), "bf16").tolist()
    assert got[:8] == [one, one, one + 2.0 ** -6, one + 2.0 ** -7, -2.5, 0.0, 2.0 ** -130, 2.0 ** -132], got
    assert got[8] == math.inf
    rng = np.random.default_rng(81)
    v32 = (rng.normal(size=4000) * np.exp(rng.uniform(-20, 20, size=4000))).astype(np.float32)
    assert np.array_equal(O.round_once(v32.astype(np.float64), "bf16"), O.round_to_act(v32, "bf16"))
    assert np.array_equal(O.round_once(v32.astype(np.float64) * (1 + 2.0 ** -40), "f32"),
                          v32.astype(np.float64))


def check_round_to_act():
    # round-to-nearest-even at the 16-bit boundary of binary32
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -7 + 2.0 ** -9, -2.5])
    got = O.round_to_act(vals, "bf16").tolist()
    assert got == [1.0, 1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -2.5]


def check_capacity_formula():
    # 0x06: T=8, k=2, E=4: CF 1.25 gives 5 slots (20 reserved, slack 4); CF 1.0 gives 4
    assert O.capacity_slots(8, 2, 4, 1.25) == 5
    assert 4 * O.capacity_slots(8, 2, 4, 1.25) - 8 * 2 == 4
    assert O.capacity_slots(8, 2, 4, 1.0) == 4
    # 0x06A group example: T_g=4, E=4, k=1, CF=1 -> one slot each; the global view has 2
    assert O.capacity_slots(4, 1, 4, 1.0) == 1 and O.capacity_slots(8, 1, 4, 1.0) == 2
    # a route budget that is not a whole number rounds up
    assert O.capacity_slots(10, 3, 7, 1.0) == 5


def check_capacity_group_example():
    # 0x06A: groups A (E0,E0,E1,E1) and B (E2,E2,E3,E3) with one slot per expert
    # drop two routes each; the same eight routes as one group with 2 slots drop none
    gates = np.array([[0.9], [0.8], [0.7], [0.6]])
    a, _ = O.arbitrate_capacity(np.array([[0], [0], [1], [1]]), gates, 1)
    b, _ = O.arbitrate_capacity(np.array([[2], [2], [3], [3]]), gates, 1)
    assert (~a).sum() == 2 and (~b).sum() == 2
    both, _ = O.arbitrate_capacity(np.array([[0], [0], [1], [1], [2], [2], [3], [3]]),
                                   np.vstack([gates, gates]), 2)
    assert both.all()


def check_capacity_focal_token():
    # 0x06A: with one slot, focal token f (gate 0.80) beats a competitor at 0.70
    # and overflows against one at 0.90, whatever its own position
    for f_first in (True, False):
        for comp, f_accepted in ((0.70, True), (0.90, False)):
            g = [[0.80], [comp]] if f_first else [[comp], [0.80]]
            acc, gap = O.arbitrate_capacity(np.array([[0], [0]]), np.array(g), 1)
            f = 0 if f_first else 1
            assert bool(acc[f, 0]) == f_accepted and bool(acc[1 - f, 0]) != f_accepted
            assert abs(gap[0] - abs(0.80 - comp)) < 1e-12


def check_capacity_ties_and_sequential_claim(seed=10):
    # equal gates: the lower token id wins, then the lower selected slot
    acc, _ = O.arbitrate_capacity(np.array([[1], [1], [1]]), np.array([[0.5], [0.5], [0.5]]), 2)
    assert acc[:, 0].tolist() == [True, True, False]
    # 0x07's sketch (all routes sorted by -gate, token, slot, claiming slots in
    # that order) accepts the same routes as the per-expert ranking of 0x06A
    rng = np.random.default_rng(seed)
    for _ in range(60):
        T, E = int(rng.integers(1, 12)), int(rng.integers(2, 6))
        K = int(rng.integers(1, E + 1))
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)])
        gates = np.round(rng.random((T, K)), 1)  # coarse: many equal gates
        C = int(rng.integers(0, T + 1))
        want = np.zeros((T, K), dtype=bool)
        counts = [0] * E
        for t, k in sorted(((t, k) for t in range(T) for k in range(K)),
                           key=lambda r: (-gates[r], r[0], r[1])):
            if counts[ids[t, k]] < C:
                counts[ids[t, k]] += 1
                want[t, k] = True
        got, _ = O.arbitrate_capacity(ids, gates, C)
        assert np.array_equal(got, want)
        c, o, src, pos = O.dispatch_accepted(ids, got, E)
        n = np.bincount(ids.reshape(-1), minlength=E)
        assert c.tolist() == np.minimum(n, C).tolist() and o[-1] == got.sum()
        assert ((pos >= 0) == got.reshape(-1)).all()
        assert np.array_equal(src[pos[pos >= 0]], np.nonzero(pos >= 0)[0])


def check_capacity_fixed_drop(seed=11):
    rng = np.random.default_rng(seed)
    p, w, x = _random_layer(rng, 12, 16, 4, 2, 8, 8, rsf=1.5)
    # with room for every route the variant is the dropless layer
    big = O.layer_forward(dict(p, capacity_factor=10.0), x, w)["out"]
    assert np.allclose(big, O.layer_forward(p, x, w)["out"], rtol=0, atol=1e-12)
    # with drops: each token keeps its accepted routes at their original
    # gates, no renormalisation, plus the shared expert (0x05F)
    q = dict(p, capacity_factor=0.5)
    got = O.layer_forward(q, x, w)["out"]
    ids, gw, _ = O.route(O.router_logits(x, w["w_router"]), w.get("bias"), 1, 1, 2, 1, 1.5)
    acc, _ = O.arbitrate_capacity(ids, gw, O.capacity_slots(12, 2, 4, 0.5))
    assert (~acc).sum() > 0
    want = O.shared_expert(x, w["w_up_shared"], w["w_down_shared"])
    for t in range(12):
        for k in range(2):
            if acc[t, k]:
                e = ids[t, k]
                want[t] += gw[t, k] * O.expert_mlp(x[t:t + 1], w["w_up"][e], w["w_down"][e])[0]
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    tm = O.token_major_forward(q, x, w)["out"]
    assert np.allclose(tm, got, rtol=0, atol=1e-12)


def check_e4m3_named_values():
    v = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    named = {0x00: 0.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x07: 7 * 2.0 ** -9, 0x01: 2.0 ** -9,
             0x38: 1.0, 0x30: 0.5, 0x40: 2.0, 0x3C: 1.5, 0xC0: -2.0, 0xFE: -448.0, 0x80: 0.0}
    for c, want in named.items():
        assert v[c] == want, (hex(c), v[c])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isnan(v).sum() == 2
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)          # codes 0x00..0x7E ascend
    assert np.array_equal(v[0x80:0xFF], -pos)  # the sign bit only negates
    # the step doubles at each binade: 8 codes per binade above the subnormals
    assert np.all(np.diff(pos[8:16]) == 2.0 ** -9) and np.all(np.diff(pos[120:127]) == 32.0)


def check_e4m3_rounding():
    fin = ~np.isnan(O.e4m3_decode(np.arange(256, dtype=np.uint8)))
    codes = np.arange(256, dtype=np.uint8)[fin]
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(codes)), codes)
    cases = {1.0625: 0x38,          # midway 1 and 1.125: to the even mantissa
             1.1875: 0x3A,          # midway 1.125 and 1.25: up to the even one
             1.07: 0x39, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, 2.5 * 2.0 ** -9: 0x02,
             464.0: 0x7E, 465.0: 0x7E, 1e6: 0x7E, -1e6: 0xFE, -0.0: 0x80, -1.0625: 0xB8}
    got = O.e4m3_encode(np.array(list(cases), dtype=np.float64))
    assert got.tolist() == list(cases.values()), [hex(g) for g in got]


def check_fp8_row_quantisation(seed=12):
    rng = np.random.default_rng(seed)
    w = O.round_to_act(rng.normal(size=(3, 40, 64)) * 0.05, "bf16")
    w[1, 5] = 0.0
    codes, s = O.quantize_rows_fp8(w)
    assert codes.shape == w.shape and s.shape == (3, 40) and s.dtype == np.float32
    deq = O.dequant_rows_fp8(codes, s)
    # each row's largest magnitude lands on +-448; an all-zero row stays zero
    amax_code = np.abs(O.e4m3_decode(codes)).max(axis=-1)
    assert np.all((amax_code == 448.0) | (s == 1.0)) and np.all(deq[1, 5] == 0)
    # error within half a step of the element's binade (relative 1/16), or a
    # subnormal step of the row's scale
    err = np.abs(deq - w)
    assert np.all(err <= np.abs(w) / 16 + s[..., None] * 2.0 ** -10 + 1e-30)
    # per output channel: rows are independent
    c2, s2 = O.quantize_rows_fp8(w[0])
    assert np.array_equal(c2, codes[0]) and np.array_equal(s2, s[0])


def check_fp8_layer(seed=13):
    rng = np.random.default_rng(seed)
    p, w, x = _random_layer(rng, 10, 16, 4, 2, 8, 8)
    q = dict(p, expert_dtype="fp8")
    got = O.layer_forward(q, x, w)["out"]
    wq = dict(w)
    for k in ("w_up", "w_down", "w_up_shared", "w_down_shared"):
        wq[k] = O.dequant_rows_fp8(*O.quantize_rows_fp8(w[k]))
    assert np.allclose(got, O.layer_forward(p, x, wq)["out"], rtol=0, atol=1e-12)
    ref = O.layer_forward(p, x, w)["out"]
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert 0 < rel < 0.1, rel  # a small, non-zero quantisation error
    assert np.allclose(O.token_major_forward(q, x, w)["out"], got, rtol=0, atol=1e-12)


def check_e2m1_values():
    """The 16 E2M1 codes: the magnitudes the OCP MX format lists, the sign
    bit only negating (code 8 is -0)."""
    v = O.e2m1_decode(np.arange(16))
    assert v[:8].tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.array_equal(v[8:], -v[:8]) and np.signbit(v[8]) and not np.signbit(v[0])


def _e2m1_nearest_brute(a):
    """E2M1 code of each value by search over the 8 magnitudes: the nearest
    one, on a tie the code with mantissa bit 0 (the even one)."""
    mags = O.e2m1_decode(np.arange(8))
    out = []
    for x in np.asarray(a, dtype=np.float64):
        dist = np.abs(abs(x) - mags)
        best = [c for c in range(8) if dist[c] == dist.min()]
        c = [b for b in best if b % 2 == 0][0] if len(best) > 1 else best[0]
        out.append(c | (8 if np.signbit(x) else 0))
    return np.array(out, dtype=np.uint8)


def check_e2m1_rounding():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(O.e2m1_encode(O.e2m1_decode(codes)), codes)
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6,  # ties: the even code
             7.0: 7, 100.0: 7, 0.2: 0, 0.3: 1, 5.01: 7, -0.0: 8, -0.3: 9, -5.0: 14, -7.5: 15}
    got = O.e2m1_encode(np.array(list(cases), dtype=np.float64))
    assert got.tolist() == list(cases.values()), got.tolist()
    grid = np.concatenate([np.linspace(-9, 9, 1441), np.arange(-8, 8.01, 0.25)])
    assert np.array_equal(O.e2m1_encode(grid), _e2m1_nearest_brute(grid))


def check_mxfp4_blocks(seed=14):
    rng = np.random.default_rng(seed)
    w = O.round_to_act(rng.normal(size=(3, 40, 64)) * 0.05, "bf16")
    w[1, 5, 32:] = 0.0                  # an all-zero block
    w[2, 7, :32] = 0.0
    w[2, 7, 3] = 0.25                   # amax a power of two: lands on 4
    w[2, 8, :32] = np.clip(w[2, 8, :32], -0.3, 0.3)
    w[2, 8, 9] = -0.4375                # amax / 2^shared = 7: saturates to 6
    codes, sc = O.quantize_blocks_mxfp4(w)
    assert codes.shape == w.shape and sc.shape == (3, 40, 2) and sc.dtype == np.uint8
    assert codes.max() <= 15
    deq = O.dequant_blocks_mxfp4(codes, sc)
    assert sc[1, 5, 1] == 0 and np.all(codes[1, 5, 32:] == 0) and np.all(deq[1, 5, 32:] == 0)
    # closed form of the shared exponent: amax / 2^shared in [4, 8)
    blk = np.abs(w).reshape(3, 40, 2, 32).max(axis=-1)
    x = np.exp2(sc.astype(np.float64) - 127)
    nz = blk > 0
    assert np.all((blk[nz] / x[nz] >= 4) & (blk[nz] / x[nz] < 8))
    assert deq[2, 7, 3] == 0.25 and codes[2, 7, 3] == 6
    assert codes[2, 8, 9] == 15 and deq[2, 8, 9] == -0.375
    # error within half a step of the element's E2M1 binade, 2 steps past 6
    xe = np.repeat(x, 32, axis=-1)
    a = np.abs(w) / xe
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, np.where(a <= 6, 1.0, 2.0)))
    assert np.all(np.abs(deq - w) <= half * xe)
    # blocks are independent and run along the last (input) axis
    c2, s2 = O.quantize_blocks_mxfp4(w[0, 3:4, 32:64])
    assert np.array_equal(c2[0], codes[0, 3, 32:]) and s2[0, 0] == sc[0, 3, 1]


def check_mxfp4_layer(seed=15):
    rng = np.random.default_rng(seed)
    p, w, x = _random_layer(rng, 10, 64, 4, 2, 32, 64)
    q = dict(p, expert_dtype="mxfp4")
    got = O.layer_forward(q, x, w)["out"]
    wq = dict(w)
    for k in ("w_up", "w_down", "w_up_shared", "w_down_shared"):
        wq[k] = O.dequant_blocks_mxfp4(*O.quantize_blocks_mxfp4(w[k]))
    assert np.allclose(got, O.layer_forward(p, x, wq)["out"], rtol=0, atol=1e-12)
    ref = O.layer_forward(p, x, w)["out"]
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert 0.01 < rel < 0.3, rel  # a 4-bit quantisation error: visible, bounded
    assert np.allclose(O.token_major_forward(q, x, w)["out"], got, rtol=0, atol=1e-12)


def check_mxfp8_blocks():
    """MXFP8 activation blocks (OCP MX E4M3, one E8M0 scale per 32 along the
    last axis): the shared exponent floor(log2 amax) - 8 puts amax / scale
    in [256, 512); magnitudes past 448 saturate; ties go to the even code in
    normal and subnormal binades; an all-zero block takes scale code 0;
    blocks are independent and run along the last axis."""
    a = np.zeros((2, 64))
    a[0, :5] = [256.0, 9.5 * 1.0, 2.0 ** -8 + 2.0 ** -10, 500.0, -3.0]   # amax 500: shared 0
    a[0, 32:35] = [1.75 * 2.0 ** 20, 2.0 ** 12 + 2.0 ** 8, -(2.0 ** 20)]  # shared 20 - 8 = 12
    codes, scales = O.quantize_blocks_mxfp8(a)
    assert scales.tolist() == [[127, 139], [0, 0]], scales
    v = O.dequant_blocks_mxfp8(codes, scales)
    assert v[0, :5].tolist() == [256.0, 10.0, 2.0 ** -8, 448.0, -3.0], v[0, :5]
    assert v[0, 32:35].tolist() == [1.75 * 2.0 ** 20, 2.0 ** 12, -(2.0 ** 20)], v[0, 32:35]
    assert np.all(v[1] == 0) and np.all(v[0, 5:32] == 0)
    # amax / scale in [256, 512) for every non-zero block; the error of each
    # element within half a step of its E4M3 binade (saturation aside)
    rng = np.random.default_rng(61)
    b = rng.normal(size=(5, 96)) * np.exp(rng.uniform(-6, 6, size=(5, 1)))
    c, sc = O.quantize_blocks_mxfp8(b)
    blk = np.abs(b.astype(np.float32).astype(np.float64)).reshape(5, 3, 32)
    ratio = blk.max(axis=-1) / np.exp2(sc.astype(np.float64) - 127)
    assert np.all((ratio >= 256) & (ratio < 512)), ratio
    deq = O.dequant_blocks_mxfp8(c, sc).reshape(5, 3, 32)
    scale = np.exp2(sc.astype(np.float64) - 127)[..., None]
    mag = np.minimum(blk / scale, 448.0)
    step = np.exp2(np.maximum(np.floor(np.log2(np.maximum(mag, 2.0 ** -12))), -6) - 3)
    err = np.abs(np.abs(deq) / scale - mag)
    assert np.all(err <= step / 2 + 1e-12), float(np.max(err / step))
    # blocks run along the last axis: scaling one block leaves the others
    b2 = b.copy()
    b2[:, :32] *= 1024.0
    c2, sc2 = O.quantize_blocks_mxfp8(b2)
    assert np.array_equal(c2[:, 32:], c[:, 32:]) and np.array_equal(sc2[:, 1:], sc[:, 1:])
    assert np.array_equal(c2[:, :32], c[:, :32]) and np.array_equal(sc2[:, 0], sc[:, 0] + 10)
    # a square matrix: each row's block takes that row's own amax
    m = rng.normal(size=(32, 32)) * np.exp2(np.arange(32))[:, None] / 2.0 ** 10
    _, scm = O.quantize_blocks_mxfp8(m)
    own = np.floor(np.log2(np.abs(m.astype(np.float32).astype(np.float64)).max(axis=1))) - 8 + 127
    assert np.array_equal(scm[:, 0].astype(np.float64), own), (scm[:4, 0], own[:4])


def check_w4a8_layer(seed=62):
    """The W4A8 layer (MXFP4 weights, MXFP8 inputs of both expert products).
    Closed form: one row through one expert whose ReLU^2 output 6.890625 is
    not an E4M3 value (its block scale 2^-6 takes it to 441, which rounds to
    448): the down product sees 7.  Exactly representable activations leave
    the W4A16 layer unchanged; random ones change it visibly but boundedly;
    the token-major schedule agrees."""
    F, d = 32, 32
    w_up = np.zeros((1, F, d))
    w_up[0, 0, 0] = 1.5                    # an MXFP4 value (block scale 2^-2, code 6)
    w_down = np.zeros((1, d, F))
    w_down[0, 3, 0] = 1.0
    x = np.zeros((1, d))
    x[0, 0] = 1.75                          # an E4M3 value
    aq = O.activation_quantiser("mxfp4_a8")
    w4 = O.quantised_expert_weights({"w_up": w_up, "w_down": w_down}, "mxfp4_a8")
    y = O.expert_mlp(x, w4["w_up"][0], w4["w_down"][0], aq)
    assert y[0, 3] == 7.0 and np.count_nonzero(y) == 1, y[0, :5]
    y16 = O.expert_mlp(x, w4["w_up"][0], w4["w_down"][0])
    assert y16[0, 3] == (1.75 * 1.5) ** 2
    rng = np.random.default_rng(seed)
    p, w, xr = _random_layer(rng, 12, 64, 4, 2, 32, 32)
    # exactly representable activations: small integers in, and up weights
    # whose products stay small integers (h in {0, 1, 4})
    xi = np.zeros_like(xr)
    xi[np.arange(12), rng.integers(0, 64, 12)] = 1.0
    wi = dict(w, w_up=rng.integers(-2, 3, size=w["w_up"].shape).astype(np.float64),
              w_up_shared=rng.integers(-2, 3, size=w["w_up_shared"].shape).astype(np.float64))
    a = O.layer_forward(dict(p, expert_dtype="mxfp4_a8"), xi, wi)["out"]
    b = O.layer_forward(dict(p, expert_dtype="mxfp4"), xi, wi)["out"]
    assert np.array_equal(a, b)
    q = dict(p, expert_dtype="mxfp4_a8")
    got = O.layer_forward(q, xr, w)["out"]
    w16 = O.layer_forward(dict(p, expert_dtype="mxfp4"), xr, w)["out"]
    rel = np.max(np.linalg.norm(got - w16, axis=1) / np.linalg.norm(w16, axis=1))
    assert 1e-3 < rel < 0.2, rel
    assert np.allclose(O.token_major_forward(q, xr, w)["out"], got, rtol=0, atol=1e-12)
    # an up product's input rows are rounded once to bf16 before their MXFP8
    # round trip (a latent layer's projection is not bf16 yet): 1.1875 -
    # 2^-10 lies below the E4M3 midpoint of 1.125 and 1.25, so from fp32 it
    # rounds to 1.125; in bf16 it is 1.1875, the midpoint itself, which goes
    # to the even code, 1.25
    v = np.array([[1.1875 - 2.0 ** -10] + [0.0] * 31])
    aq = O.activation_quantiser("mxfp4_a8", "bf16")
    assert aq(v, "in")[0, 0] == 1.25 and aq(v, "hidden")[0, 0] == 1.125


def check_prenorm_residual(seed=9):
    rng = np.random.default_rng(seed)
    p, w, x = _random_layer(rng, 10, 16, 4, 2, 8, 8)
    w = dict(w, w_norm=1.0 + 0.1 * rng.normal(size=16))
    q = dict(p, prenorm_residual=1, norm_eps=1e-5, act_dtype="f32")
    got = O.layer_forward(q, x, w)["out"]
    xn = O.rms_norm(x, w["w_norm"], 1e-5, "f32")
    want = O.layer_forward(p, xn, w)["out"] + x
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    tm = O.token_major_forward(q, x, w)["out"]
    assert np.allclose(tm, got, rtol=0, atol=1e-12)


def _fd_gradients(p, x, w, dY, coords_per_tensor=None, seed=0, h=1e-6):
    """Central differences of L = <dY, layer_forward(x, w)> at every
    coordinate of x and of every weight (or a seeded sample of them)."""
    rng = np.random.default_rng(seed)

    def loss(xx, ww):
        return float(np.sum(dY * O.layer_forward(p, xx, ww)["out"]))

    out = {}
    tensors = {"x": x, **{k: v for k, v in w.items() if v is not None}}
    for name, t in tensors.items():
        idxs = list(np.ndindex(t.shape))
        if coords_per_tensor and len(idxs) > coords_per_tensor:
            idxs = [idxs[i] for i in rng.choice(len(idxs), coords_per_tensor, replace=False)]
        g = {}
        for idx in idxs:
            tp, tm = t.copy(), t.copy()
            tp[idx] += h
            tm[idx] -= h
            if name == "x":
                g[idx] = (loss(tp, w) - loss(tm, w)) / (2 * h)
            else:
                g[idx] = (loss(x, dict(w, **{name: tp})) - loss(x, dict(w, **{name: tm}))) / (2 * h)
        out[name] = g
    return out


_GRAD_OF = {"x": "dx", "w_router": "dw_router", "w_up": "dw_up", "w_down": "dw_down",
            "w_up_shared": "dw_up_shared", "w_down_shared": "dw_down_shared", "w_norm": "dw_norm",
            "w_latent_in": "dw_latent_in", "w_latent_out": "dw_latent_out"}


def _check_backward_fd(p, x, w, dY, tol=1e-6):
    info = O.layer_forward(p, x, w)["route_info"]
    assert info["gap"].min() > 1e-4, "the case must keep its ids under the perturbation"
    g = O.layer_backward(p, x, w, dY)
    fd = _fd_gradients(p, x, w, dY)
    for name, coords in fd.items():
        if name == "bias":
            # selection only: no gradient reaches the correction bias
            assert max(abs(v) for v in coords.values()) < tol
            continue
        an = g[_GRAD_OF[name]]
        err = max(abs(an[idx] - v) for idx, v in coords.items())
        scale = max(1.0, float(np.max(np.abs(an))))
        assert err <= tol * scale, (name, err, scale)
    return g


def _f64_layer(rng, *a, **kw):
    p, w, x = _random_layer(rng, *a, **kw)
    w = {k: np.asarray(v, dtype=np.float64) for k, v in w.items()}
    return p, w, x


def check_backward_finite_differences(seed=21):
    """Every gradient of the layer (x, router, routed and shared expert
    weights; the bias gets none) against central differences of the forward
    oracle, normalised gates, one group."""
    rng = np.random.default_rng(seed)
    p, w, x = _f64_layer(rng, 6, 8, 6, 2, 5, 4, rsf=2.5)
    dY = rng.normal(size=x.shape)
    _check_backward_fd(p, x, w, dY)


def check_backward_variants(seed=23):
    """Unnormalised gates with group-limited routing, and a capacity-bounded
    layer with dropped routes: central differences again; a dropped route
    has q = 0 but its logit still gets -s(1-s) sum_j g_j q_j / S (it stays in
    the normaliser, as [M6.1] 0x06F.3 points out for the selected softmax)."""
    rng = np.random.default_rng(seed)
    p, w, x = _f64_layer(rng, 6, 8, 8, 3, 4, 0, n_group=4, topk_group=2, rsf=1.5)
    p["norm_topk_prob"] = 0
    _check_backward_fd(p, x, w, rng.normal(size=x.shape))
    p, w, x = _f64_layer(rng, 8, 6, 4, 2, 5, 3, rsf=2.0)
    p["capacity_factor"] = 0.5
    dY = rng.normal(size=x.shape)
    r = O.layer_forward(p, x, w)
    _, margin = O.arbitrate_capacity(r["ids"], r["weights"], O.capacity_slots(8, 2, 4, 0.5))
    assert np.min(margin) > 1e-4, "the arbitration must not flip under the perturbation"
    g = _check_backward_fd(p, x, w, dY)
    rp = np.asarray(g["forward"]["route_pos"]).reshape(8, 2)
    dropped = rp < 0
    assert dropped.any() and not dropped.all()
    s = O.sigmoid(g["forward"]["logits"])
    s_sel = np.take_along_axis(s, g["forward"]["ids"].astype(np.int64), axis=1)
    gw, q = g["forward"]["weights"], g["q"]
    qbar = (gw * q).sum(axis=1, keepdims=True)
    want = -s_sel * (1 - s_sel) * qbar / s_sel.sum(axis=1, keepdims=True)
    assert np.all(q[dropped] == 0)
    assert np.allclose(g["dz"][dropped], want[dropped], rtol=1e-12, atol=0)
    assert np.any(np.abs(g["dz"][dropped]) > 1e-6)


def check_backward_invariants(seed=24):
    """Normalised gates are invariant to scaling every selected score by one
    factor, so sum_k s_k dL/ds_k = 0 per token; the gradients are linear in
    dY; a shared-expert-only layer (router weights zero... the routed part
    scaled to zero) leaves the routed weights without gradient."""
    rng = np.random.default_rng(seed)
    p, w, x = _f64_layer(rng, 7, 8, 6, 3, 5, 4, rsf=2.5)
    d1, d2 = rng.normal(size=x.shape), rng.normal(size=x.shape)
    g1, g2 = O.layer_backward(p, x, w, d1), O.layer_backward(p, x, w, d2)
    g12 = O.layer_backward(p, x, w, d1 + 2 * d2)
    for k in ("dx", "dw_router", "dw_up", "dw_down", "dw_up_shared", "dw_down_shared"):
        assert np.allclose(g12[k], g1[k] + 2 * g2[k], rtol=1e-10, atol=1e-12), k
    s = O.sigmoid(g1["forward"]["logits"])
    s_sel = np.take_along_axis(s, g1["forward"]["ids"].astype(np.int64), axis=1)
    ds = g1["dz"] / (s_sel * (1 - s_sel))
    assert np.allclose((s_sel * ds).sum(axis=1), 0.0, atol=1e-12)
    # unselected experts and zero-hit experts receive no gradient
    hits = np.bincount(g1["forward"]["ids"].reshape(-1), minlength=6)
    for e in np.nonzero(hits == 0)[0]:
        assert not g1["dw_up"][e].any() and not g1["dw_down"][e].any() and not g1["dw_router"][e].any()
    p0 = dict(p, routed_scaling_factor=0.0)
    g0 = O.layer_backward(p0, x, w, d1)
    assert not g0["dw_up"].any() and not g0["dw_down"].any() and not g0["dw_router"].any()


def check_rms_norm_backward(seed=25):
    """The norm's gradients against central differences of its definition
    (``rms_norm_exact``, eps > 0), and the facts the scale invariance of an
    eps-free RMSNorm fixes: the input gradient is orthogonal to the row
    (<h, dh> = 0), scales as 1 / alpha when the row is scaled by alpha, and
    vanishes for dx = n with w = 1 (L = |n|^2 / 2 = d / 2 is constant)."""
    rng = np.random.default_rng(seed)
    T, d, eps = 3, 7, 0.3
    h = rng.normal(size=(T, d))
    w = 1.0 + 0.2 * rng.normal(size=d)
    dX = rng.normal(size=(T, d))
    dh, dw = O.rms_norm_backward(h, w, eps, dX)
    loss = lambda hh, ww: float(np.sum(dX * O.rms_norm_exact(hh, ww, eps)))
    e = 1e-6
    for t in range(T):
        for j in range(d):
            hp, hm = h.copy(), h.copy()
            hp[t, j] += e
            hm[t, j] -= e
            assert abs((loss(hp, w) - loss(hm, w)) / (2 * e) - dh[t, j]) < 1e-7
    for j in range(d):
        wp, wm = w.copy(), w.copy()
        wp[j] += e
        wm[j] -= e
        assert abs((loss(h, wp) - loss(h, wm)) / (2 * e) - dw[j]) < 1e-7
    dh0, _ = O.rms_norm_backward(h, w, 0.0, dX)
    assert np.allclose((h * dh0).sum(axis=1), 0.0, atol=1e-12)
    dh3, _ = O.rms_norm_backward(3.0 * h, w, 0.0, dX)
    assert np.allclose(dh3, dh0 / 3.0, rtol=1e-12, atol=1e-14)
    n = O.rms_norm_exact(h, np.ones(d), 0.0)
    dhn, _ = O.rms_norm_backward(h, np.ones(d), 0.0, n)
    assert np.allclose(dhn, 0.0, atol=1e-13)


def check_backward_prenorm_finite_differences(seed=26):
    """The layer with the fused front and back (the input is the hidden
    state H, out = Y + H): every gradient, the norm weight's included,
    against central differences of the forward oracle (no rounding of the
    normed rows, act_dtype "f64", so the differences see the definition)."""
    rng = np.random.default_rng(seed)
    p, w, x = _f64_layer(rng, 6, 8, 6, 2, 5, 4, rsf=2.5)
    w["w_norm"] = 1.0 + 0.2 * rng.normal(size=8)
    p.update(prenorm_residual=1, norm_eps=1e-3, act_dtype="f64")
    dY = rng.normal(size=x.shape)
    g = _check_backward_fd(p, x, w, dY)
    assert g["dw_norm"] is not None and g["dw_norm"].shape == (8,)


def check_backward_latent_finite_differences(seed=27):
    """A latent layer (router and shared expert on x, routed experts on
    x W_lin^T, out = y_lat W_lout^T + y_s): every gradient, both projections'
    included, against central differences of the forward oracle; with a
    shared expert and without."""
    rng = np.random.default_rng(seed)
    for Fs in (4, 0):
        p, w, x = _f64_layer(rng, 6, 8, 6, 2, 5, Fs, rsf=2.5, latent=5)
        w["w_latent_in"] = rng.normal(scale=8 ** -0.5, size=(5, 8))
        w["w_latent_out"] = rng.normal(scale=5 ** -0.5, size=(8, 5))
        dY = rng.normal(size=x.shape)
        g = _check_backward_fd(p, x, w, dY)
        assert g["dw_latent_in"].shape == (5, 8) and g["dw_latent_out"].shape == (8, 5)
        assert g["dw_up"].shape == (6, 5, 5) and g["dw_down"].shape == (6, 5, 5)


def check_backward_latent_conjugation(seed=28):
    """The latent layer that equals the plain one (W_lin = 2 P, W_lout =
    P^T / 4, experts conjugated by a non-symmetric permutation P, as in
    check_latent_orientation) has the plain layer's input, router and
    shared-expert gradients.  For any expert weights W', that layer's
    output is the plain layer's with W_up = W'_up P and W_down = P^T
    W'_down (ReLU^2 is homogeneous of degree 2: the factor 2 of W_lin gives
    4 in the hidden, which W_lout's 1/4 takes back), so by the chain rule its
    expert gradients are the plain ones carried through those maps: dW_up P^T
    and P dW_down."""
    rng = np.random.default_rng(seed)
    d = 8
    p, w, x = _f64_layer(rng, 9, d, 6, 2, 5, 4, rsf=2.5, latent=d)
    P = np.roll(np.eye(d), 1, axis=0)
    P[[0, 3]] = P[[3, 0]]
    assert not np.allclose(P, P.T)
    wl = dict(w, w_latent_in=2.0 * P, w_latent_out=0.25 * P.T,
              w_up=np.stack([u @ P.T for u in w["w_up"]]), w_down=np.stack([P @ dn for dn in w["w_down"]]))
    dY = rng.normal(size=x.shape)
    gp = O.layer_backward(dict(p, d_latent=0), x, w, dY)
    gl = O.layer_backward(p, x, wl, dY)
    for k in ("dx", "dw_router", "dw_up_shared", "dw_down_shared"):
        assert np.allclose(gl[k], gp[k], rtol=1e-10, atol=1e-12), k
    for e in range(6):
        assert np.allclose(gl["dw_up"][e], gp["dw_up"][e] @ P.T, rtol=1e-10, atol=1e-12)
        assert np.allclose(gl["dw_down"][e], P @ gp["dw_down"][e], rtol=1e-10, atol=1e-12)


ALL_CHECKS = [check_selection_brute_force, check_sigmoid_closed_forms, check_decision_scores,
              check_router_orientation, check_token_choice_table, check_group_score_is_top2_sum,
              check_masked_groups_never_selected, check_tie_rules, check_decision_in_fp32,
              check_weights, check_dispatch_fixture, check_dispatch_round_trip,
              check_combine_trace, check_dense_equivalent, check_token_major_matches_expert_major,
              check_latent_scaling, check_latent_orientation, check_accumulate_out, check_relu2,
              check_relu2_zero_fraction, check_boundary_gap_closed_forms,
              check_rms_norm_worked_example, check_rms_norm_constant_row,
              check_rms_norm_rounds_once, check_round_once, check_round_to_act, check_prenorm_residual,
              check_capacity_formula, check_capacity_group_example, check_capacity_focal_token,
              check_capacity_ties_and_sequential_claim, check_capacity_fixed_drop,
              check_e4m3_named_values, check_e4m3_rounding, check_fp8_row_quantisation, check_fp8_layer,
              check_e2m1_values, check_e2m1_rounding, check_mxfp4_blocks, check_mxfp4_layer,
              check_mxfp8_blocks, check_w4a8_layer,
              check_backward_finite_differences, check_backward_variants, check_backward_invariants,
              check_rms_norm_backward, check_backward_prenorm_finite_differences,
              check_backward_latent_finite_differences, check_backward_latent_conjugation]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()


# ---------------------------------------------------------------------------
# planted mistakes (on the CPU, in the oracle): each must fail a pin
# ---------------------------------------------------------------------------

@contextlib.contextmanager
def patched(name, fn):
    orig = getattr(O, name)
    setattr(O, name, fn)
    try:
        yield orig
    finally:
        setattr(O, name, orig)


def _mut_weights_from_corrected():
    orig = O.decision_scores

    def f(logits, bias):
        s64, s32, c32, c64 = orig(logits, bias)
        return c64, s32, c32, c64
    return "decision_scores", f


def _mut_group_by_max():
    def f(c, n_group):
        T, E = c.shape
        return c.reshape(T, n_group, E // n_group).max(axis=-1)
    return "group_scores", f


def _mut_high_id_ties():
    def f(c32, eligible, K):
        E = c32.shape[1]
        key = np.where(eligible, -c32.astype(np.float64), np.inf)
        order = np.argsort(key[:, ::-1], axis=1, kind="stable")
        return (E - 1 - order[:, :K]).astype(np.int32)
    return "select_experts", f


def _mut_unstable_ties():
    def f(c32, eligible, K):
        key = np.where(eligible, -c32.astype(np.float64), np.inf)
        return np.argsort(key, axis=1, kind="heapsort")[:, :K].astype(np.int32)  # not stable
    return "select_experts", f


def _mut_no_norm():
    orig = O.gate_weights
    return "gate_weights", lambda s64, ids, norm, rsf: orig(s64, ids, 0, rsf)


def _mut_scale_before_norm():
    def f(s64, ids, norm, rsf):
        w = np.take_along_axis(s64, ids.astype(np.int64), axis=1) * rsf
        if norm:
            w = w / w.sum(axis=1, keepdims=True)
        return w
    return "gate_weights", f


def _mut_zero_mask():
    def f(c32, eligible, K):
        key = np.where(eligible, -c32.astype(np.float64), 0.0)
        return np.argsort(key, axis=1, kind="stable")[:, :K].astype(np.int32)
    return "select_experts", f


def _mut_overwrite_combine():
    def f(y_packed, weights, ids, route_pos, y_shared=None, out_prev=None):
        T, K = ids.shape
        rp = np.asarray(route_pos).reshape(T, K)
        out = np.zeros((T, y_packed.shape[1]))
        for t in range(T):
            for k in np.argsort(ids[t]):
                out[t] = weights[t, k] * y_packed[rp[t, k]]
        if y_shared is not None:
            out += y_shared
        if out_prev is not None:
            out += out_prev
        return out
    return "combine", f


def _mut_residual_in_combine():
    orig = O.combine

    def f(y_packed, weights, ids, route_pos, y_shared=None, out_prev=None):
        out = orig(y_packed, weights, ids, route_pos, y_shared, out_prev)
        return out + 1.0  # anything added outside the routed sum
    return "combine", f


def _mut_wrong_slot_gate():
    orig = O.combine

    def f(y_packed, weights, ids, route_pos, y_shared=None, out_prev=None):
        return orig(y_packed, np.asarray(weights)[:, ::-1], ids, route_pos, y_shared, out_prev)
    return "combine", f


def _mut_drop_route():
    orig = O.dispatch

    def f(ids, E):
        counts, offsets, route_src, route_pos = orig(ids, E)
        route_pos = route_pos.copy()
        route_pos[0] = route_pos[1]  # route 0 reads route 1's packed row
        return counts, offsets, route_src, route_pos
    return "dispatch", f


def _mut_unsorted_pack():
    orig = O.dispatch

    def f(ids, E):
        counts, offsets, route_src, route_pos = orig(ids, E)
        rs = route_src.copy()
        if offsets[1] - offsets[0] >= 2:
            rs[0], rs[1] = rs[1], rs[0]
        rp = np.empty_like(route_pos)
        rp[rs] = np.arange(len(rs))
        return counts, offsets, rs, rp
    return "dispatch", f


def _mut_router_on_latent():
    orig = O.router_logits

    def f(x, w_router):
        return 2.0 * orig(x, w_router)  # as if routed from the 2x latent input
    return "router_logits", f


def _mut_no_relu():
    return "relu2", lambda u: np.asarray(u, dtype=np.float64) ** 2


def _mut_sigmoid_wrong_sign():
    return "sigmoid", lambda z: 1.0 / (1.0 + np.exp(np.asarray(z, dtype=np.float64)))


def _mut_bias_ignored():
    orig = O.decision_scores
    return "decision_scores", lambda logits, bias: orig(logits, None)


def _mut_transposed_down():
    def f(x_rows, w_up_e, w_down_e, act_q=None):
        h = O.relu2(np.asarray(x_rows) @ np.asarray(w_up_e).T)
        return h @ np.asarray(w_up_e)  # the up matrix, transposed, as the down projection
    return "expert_mlp", f


def _mut_rms_sum_not_mean():
    orig = O.rms_norm

    def f(h, w_norm, eps, act_dtype):
        d = np.asarray(h).shape[1]
        return orig(np.asarray(h) / math.sqrt(d), w_norm, eps, act_dtype)  # sum of squares, no mean
    return "rms_norm", f


def _mut_rms_one_plus_w():
    orig = O.rms_norm
    return "rms_norm", lambda h, w_norm, eps, act: orig(h, 1.0 + np.asarray(w_norm), eps, act)


def _mut_rms_eps_outside():
    orig = O.rms_norm

    def f(h, w_norm, eps, act_dtype):
        return orig(h, w_norm, 0.0, act_dtype)  # eps ignored
    return "rms_norm", f


def _mut_no_residual():
    orig = O._front

    def f(p, x, w, out_prev):
        xn, _ = orig(p, x, w, out_prev)
        return xn, out_prev
    return "_front", f


def _mut_capacity_floor():
    return "capacity_slots", lambda T, K, E, cf: int(math.floor(float(cf) * T * K / E))


def _mut_arbitration_source_order():
    orig = O.arbitrate_capacity
    return "arbitrate_capacity", lambda ids, gates, C: orig(ids, np.zeros_like(np.asarray(gates, float)), C)


def _mut_arbitration_ascending_gate():
    orig = O.arbitrate_capacity
    return "arbitrate_capacity", lambda ids, gates, C: orig(ids, -np.asarray(gates, float), C)


def _mut_renormalise_after_drop():
    orig = O.combine

    def f(y_packed, weights, ids, route_pos, y_shared=None, out_prev=None):
        rp = np.asarray(route_pos).reshape(np.asarray(ids).shape)
        w = np.where(rp >= 0, np.asarray(weights, float), 0.0)
        full = np.asarray(weights, float).sum(axis=1, keepdims=True)
        kept = w.sum(axis=1, keepdims=True)
        w = w * np.where(kept > 0, full / np.where(kept > 0, kept, 1.0), 1.0)
        return orig(y_packed, w, ids, route_pos, y_shared, out_prev)
    return "combine", f


def _mut_e4m3_no_subnormals():
    orig = O.e4m3_decode

    def f(codes):
        c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
        v = orig(codes)
        e, m = (c >> 3) & 0xF, c & 0x7
        sub = (e == 0) & (m > 0)
        return np.where(sub, np.where(c & 0x80, -1.0, 1.0) * (1 + m / 8.0) * 2.0 ** -7, v)
    return "e4m3_decode", f


def _mut_e4m3_truncate():
    orig = O.e4m3_encode

    def f(v):
        v = np.asarray(v, dtype=np.float32).astype(np.float64)
        a = np.abs(v)
        e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6.0)
        q = np.exp2(e - 3.0)
        return orig(np.sign(v) * np.floor(a / q) * q)
    return "e4m3_encode", f


def _mut_fp8_scale_amax():
    orig = O.quantize_rows_fp8

    def f(w):
        codes, s = orig(np.asarray(w) / 448.0)
        return codes, (s * np.float32(448.0)).astype(np.float32)
    return "quantize_rows_fp8", f


def _mut_fp8_per_column():
    orig = O.quantize_rows_fp8

    def f(w):
        w = np.asarray(w)
        if w.ndim < 2:
            return orig(w)
        c, s = orig(np.swapaxes(w, -1, -2))
        s_full = np.broadcast_to(s[..., :1], w.shape[:-1]).astype(np.float32)
        return np.swapaxes(c, -1, -2), s_full
    return "quantize_rows_fp8", f


def _mut_e2m1_truncate():
    orig = O.e2m1_encode

    def f(v):
        v = np.asarray(v, dtype=np.float64)
        a = np.abs(v)
        e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), 0.0)
        q = np.exp2(e - 1.0)
        return orig(np.where(np.signbit(v), -1.0, 1.0) * np.floor(a / q) * q)
    return "e2m1_encode", f


def _mut_e2m1_ties_away():
    orig = O.e2m1_encode

    def f(v):
        v = np.asarray(v, dtype=np.float64)
        a = np.abs(v)
        e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), 0.0)
        q = np.exp2(e - 1.0)
        return orig(np.where(np.signbit(v), -1.0, 1.0) * np.floor(a / q + 0.5) * q)
    return "e2m1_encode", f


def _mut_mx_shared_exponent():
    orig = O.quantize_blocks_mxfp4

    def f(w):
        codes, sc = orig(np.asarray(w, dtype=np.float64) * 2.0)  # floor(log2 amax) - 1
        return codes, (sc.astype(np.int64) - 1).astype(np.uint8)
    return "quantize_blocks_mxfp4", f


def _mut_mx_blocks_along_rows():
    orig = O.quantize_blocks_mxfp4

    def f(w):
        w = np.asarray(w, dtype=np.float64)
        if w.ndim < 2 or w.shape[-2] % 32:
            return orig(w)
        c, sc = orig(np.swapaxes(w, -1, -2))
        # one scale per 32 rows, repeated over the columns' blocks
        c = np.swapaxes(c, -1, -2)
        s_rows = np.swapaxes(sc, -1, -2)  # [..., R/32, C]
        s_new = s_rows[..., :, ::32]
        s_new = np.repeat(s_new, 32, axis=-2)[..., :w.shape[-2], :]
        return c, s_new.astype(np.uint8)
    return "quantize_blocks_mxfp4", f


def _mut_bwd_no_normaliser_term():
    orig = O.gate_backward

    def f(s_sel, q, norm, rsf):
        s_sel = np.asarray(s_sel, dtype=np.float64)
        S = s_sel.sum(axis=1, keepdims=True) if norm else 1.0
        return float(rsf) * np.asarray(q) / S * s_sel * (1.0 - s_sel)  # the sum_j g_j q_j term dropped
    return "gate_backward", f


def _mut_bwd_sigmoid_slope():
    orig = O.gate_backward

    def f(s_sel, q, norm, rsf):
        s_sel = np.asarray(s_sel, dtype=np.float64)
        return orig(s_sel, q, norm, rsf) / (1.0 - s_sel)
    return "gate_backward", f


def _mut_bwd_relu_not_relu2():
    def f(x_rows, w_up_e, w_down_e, dU):
        x_rows = np.asarray(x_rows, dtype=np.float64)
        u = x_rows @ np.asarray(w_up_e).T
        a = np.maximum(u, 0.0)
        du = (np.asarray(dU) @ np.asarray(w_down_e)) * (u > 0)
        return {"dx": du @ np.asarray(w_up_e), "dw_up": du.T @ x_rows, "dw_down": np.asarray(dU).T @ (a * a)}
    return "expert_backward", f


def _mut_bwd_transposed_dw_down():
    orig = O.expert_backward

    def f(x_rows, w_up_e, w_down_e, dU):
        g = orig(x_rows, w_up_e, w_down_e, dU)
        dwd = g["dw_down"]
        if dwd.shape[0] == dwd.shape[1]:
            g["dw_down"] = dwd.T
        else:
            g["dw_down"] = dwd[::-1]
        return g
    return "expert_backward", f


def _mut_bwd_no_router_path():
    orig = O.layer_backward

    def f(p, x, w, dY):
        g = orig(p, x, w, dY)
        GZ = np.zeros((np.asarray(x).shape[0], p["E"]))
        for t in range(GZ.shape[0]):
            for k in range(p["K"]):
                GZ[t, g["forward"]["ids"][t, k]] += g["dz"][t, k]
        g["dx"] = g["dx"] - GZ @ np.asarray(w["w_router"], dtype=np.float64)
        return g
    return "layer_backward", f


def _mut_bwd_overwrite_scatter():
    def f(dx, toks, dx_rows):
        for i, t in enumerate(toks):
            dx[t] = dx_rows[i]
        return dx
    return "gather_adjoint", f


def _mut_rms_double_rounding():
    # float64 -> fp32 -> bfloat16: two roundings instead of one
    return "round_once", lambda v, act: O.round_to_act(np.asarray(v, dtype=np.float64), act)


def _mut_rms_eps_outside_root():
    def f(h, w_norm, eps):
        h = np.asarray(h, dtype=np.float64)
        ms = np.mean(h * h, axis=1)
        return h / (np.sqrt(ms) + eps)[:, None] * np.asarray(w_norm)[None, :]
    return "rms_norm_exact", f


def _mut_gap_halved():
    orig = O._boundary_info

    def f(*a, **k):
        info = orig(*a, **k)
        return dict(info, gap=info["gap"] / 2)
    return "_boundary_info", f


def _mut_gap_no_group_term():
    orig = O._boundary_info

    def f(logits, bias, c32, c64, elig, ids, n_group, topk_group, K):
        return orig(logits, bias, c32, c64, elig, ids, 1, 1, K)
    return "_boundary_info", f


def _mut_latent_in_transposed():
    orig = O.layer_forward

    def f(p, x, w, out_prev=None):
        if w.get("w_latent_in") is not None:
            w = dict(w, w_latent_in=np.asarray(w["w_latent_in"]).T)
        return orig(p, x, w, out_prev)
    return "layer_forward", f


def _mut_latent_out_transposed():
    orig = O.layer_forward

    def f(p, x, w, out_prev=None):
        if w.get("w_latent_out") is not None:
            w = dict(w, w_latent_out=np.asarray(w["w_latent_out"]).T)
        return orig(p, x, w, out_prev)
    return "layer_forward", f


def _mut_zero_fraction_counts_negative():
    return "relu2_zero_fraction", lambda h: float(np.count_nonzero(np.asarray(h) < 0)) / max(np.asarray(h).size, 1)


def _mut_mx8_emax():
    # shared exponent floor(log2 amax) - 7: amax lands in [128, 256)
    def f(a):
        a32 = np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)
        shp = a32.shape
        blk = a32.reshape(shp[:-1] + (shp[-1] // 32, 32))
        amax = np.max(np.abs(blk), axis=-1)
        with np.errstate(divide="ignore"):
            lg = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
        sh = np.where(amax > 0, np.clip(lg - 7, -127, 127), -127.0)
        return O.e4m3_encode(blk / np.exp2(sh)[..., None]).reshape(shp), (sh + 127).astype(np.uint8)
    return "quantize_blocks_mxfp8", f


def _mut_mx8_down_input_unquantised():
    orig = O.expert_mlp

    def f(x_rows, w_up_e, w_down_e, act_q=None):
        x_rows = np.asarray(x_rows, dtype=np.float64)
        if act_q is not None:
            x_rows = act_q(x_rows, "in")
        return orig(x_rows, w_up_e, w_down_e, None)
    return "expert_mlp", f


def _mut_mx8_latent_input_unrounded():
    # the latent rows quantised from their float64 values, not the bf16 rows
    orig = O.activation_quantiser

    def f(expert_dtype, act_dtype="bf16"):
        aq = orig(expert_dtype, "f32")
        return aq
    return "activation_quantiser", f


def _mut_mx8_blocks_along_rows():
    orig = O.quantize_blocks_mxfp8

    def f(a):
        a = np.asarray(a, dtype=np.float64)
        if a.ndim < 2 or a.shape[-2] % 32:
            return orig(a)
        c, s = orig(np.swapaxes(a, -1, -2))
        return np.swapaxes(c, -1, -2), s
    return "quantize_blocks_mxfp8", f


def _mut_rms_bwd_no_projection():
    def f(h, w_norm, eps, dx):
        h = np.asarray(h, dtype=np.float64)
        r = np.sqrt(np.mean(h * h, axis=1) + float(eps))[:, None]
        return np.asarray(dx) * np.asarray(w_norm)[None, :] / r, (np.asarray(dx) * h / r).sum(axis=0)
    return "rms_norm_backward", f  # the mean(n * dn) term dropped


def _mut_rms_bwd_dw_halved():
    orig = O.rms_norm_backward

    def f(h, w_norm, eps, dx):
        dh, dw = orig(h, w_norm, eps, dx)
        return dh, 0.5 * dw  # the norm weight's gradient halved
    return "rms_norm_backward", f


def _mut_prenorm_bwd_no_residual():
    orig = O.layer_backward

    def f(p, x, w, dY):
        g = orig(p, x, w, dY)
        if p.get("prenorm_residual"):
            g = dict(g, dx=g["dx"] - np.asarray(dY, dtype=np.float64))  # out = Y + H's path to H dropped
        return g
    return "layer_backward", f


def _mut_latent_bwd_dw_lout_wrong_operand():
    orig = O.layer_backward

    def f(p, x, w, dY):
        g = orig(p, x, w, dY)
        if p.get("d_latent") and not p.get("prenorm_residual"):
            x_lat = np.asarray(x, dtype=np.float64) @ np.asarray(w["w_latent_in"], dtype=np.float64).T
            g = dict(g, dw_latent_out=np.asarray(dY, dtype=np.float64).T @ x_lat)  # x_lat for y_lat
        return g
    return "layer_backward", f


def _mut_latent_bwd_input_path_dropped():
    orig = O.layer_backward

    def f(p, x, w, dY):
        g = orig(p, x, w, dY)
        if p.get("d_latent") and not p.get("prenorm_residual"):
            # keep only the router's and the shared expert's parts of dx
            fw = g["forward"]
            x64 = np.asarray(x, dtype=np.float64)
            GZ = np.zeros((x64.shape[0], p["E"]))
            for t in range(x64.shape[0]):
                for k in range(p["K"]):
                    GZ[t, fw["ids"][t, k]] += g["dz"][t, k]
            dx = GZ @ np.asarray(w["w_router"], dtype=np.float64)
            if p.get("F_shared", 0):
                dx = dx + O.expert_backward(x64, w["w_up_shared"], w["w_down_shared"], dY)["dx"]
            g = dict(g, dx=dx)
        return g
    return "layer_backward", f


MUTATIONS = [_mut_mx8_emax, _mut_mx8_down_input_unquantised, _mut_mx8_blocks_along_rows,
             _mut_mx8_latent_input_unrounded,
             _mut_rms_double_rounding, _mut_rms_eps_outside_root, _mut_gap_halved, _mut_gap_no_group_term,
             _mut_latent_in_transposed, _mut_latent_out_transposed, _mut_zero_fraction_counts_negative,
             _mut_bwd_no_normaliser_term, _mut_bwd_sigmoid_slope, _mut_bwd_relu_not_relu2,
             _mut_bwd_transposed_dw_down, _mut_bwd_no_router_path, _mut_bwd_overwrite_scatter,
             _mut_e4m3_no_subnormals, _mut_e4m3_truncate, _mut_fp8_scale_amax, _mut_fp8_per_column,
             _mut_e2m1_truncate, _mut_e2m1_ties_away, _mut_mx_shared_exponent, _mut_mx_blocks_along_rows,
             _mut_capacity_floor, _mut_arbitration_source_order, _mut_arbitration_ascending_gate,
             _mut_renormalise_after_drop, _mut_rms_sum_not_mean, _mut_rms_one_plus_w, _mut_rms_eps_outside, _mut_no_residual,
             _mut_weights_from_corrected, _mut_group_by_max, _mut_high_id_ties,
             _mut_unstable_ties, _mut_no_norm, _mut_scale_before_norm, _mut_zero_mask,
             _mut_overwrite_combine, _mut_residual_in_combine, _mut_wrong_slot_gate,
             _mut_drop_route, _mut_unsorted_pack, _mut_router_on_latent, _mut_no_relu,
             _mut_sigmoid_wrong_sign, _mut_bias_ignored, _mut_transposed_down,
             _mut_rms_bwd_no_projection, _mut_rms_bwd_dw_halved, _mut_prenorm_bwd_no_residual,
             _mut_latent_bwd_dw_lout_wrong_operand, _mut_latent_bwd_input_path_dropped]


@pytest.mark.parametrize("mut", MUTATIONS, ids=lambda f: f.__name__)
def test_mutations_are_caught(mut):
    name, fn = mut()
    failed = []
    with patched(name, fn):
        for check in ALL_CHECKS:
            try:
                check()
            except (AssertionError, ValueError):
                # every pin passes on the oracle as written (test_oracle_pin),
                # so a pin that fails, or that a planted shape error stops,
                # has caught the mistake
                failed.append(check.__name__)
    assert failed, "planted mistake %s passed every pin" % mut.__name__
