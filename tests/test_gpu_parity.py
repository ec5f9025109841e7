"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar: ids, counts, offsets and the route maps bit-exact (rows whose router
boundary gap is below 1e-5 are counted as near-ties and re-checked with the
GPU's own choice); outputs within 2e-2 (bf16) or 1e-4 (fp32) by both the
max row-relative L2 error and the max per-row element error (max |dy| over
the row's max |y|); repeated runs bitwise identical.  The fused layer is
checked on its own routing, read from its workspace.
"""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
import routed_relu_expert_amd as M
from routed_relu_expert_amd import synth

from . import _harness as H

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DEV = "cuda"


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _np(t):
    return t.detach().cpu().numpy()


# ---------------------------------------------------------------------------
# page fixtures through the staged calls
# ---------------------------------------------------------------------------

def test_token_choice_table():
    g = _golden("m61_token_choice_top2.json")
    z = torch.tensor(g["affinity"], dtype=torch.float32, device=DEV)
    ids, w = M.moe_route(z, None, K=2)
    counts, offsets, rs, rp = M.moe_dispatch(ids, 4)
    torch.cuda.synchronize()
    assert _np(ids).tolist() == g["top2"]
    assert _np(counts).tolist() == g["routes_per_expert"]
    assert _np(offsets).tolist() == [0, 6, 11, 14, 16]
    assert np.allclose(_np(w).sum(1), 1.0, atol=1e-6)


def test_dispatch_route_table():
    g = _golden("m61_dispatch_route_table.json")
    ids = torch.tensor(g["expert_of_route"], dtype=torch.int32, device=DEV)
    counts, offsets, rs, rp = M.moe_dispatch(ids, g["E"])
    torch.cuda.synchronize()
    assert _np(rs).tolist() == g["packed_route_ids"]
    assert _np(offsets).tolist() == g["offsets"]
    assert np.array_equal(_np(rs)[_np(rp)], np.arange(6))


def test_combine_trace():
    g = _golden("m61_combine_trace.json")
    H_ = np.array(g["H"], dtype=np.float64)
    ids = np.array(g["expert_of_route"], dtype=np.int32)
    gates = np.array(g["gate_of_route"], dtype=np.float32)
    ex = g["experts"]
    _, _, route_src, route_pos = O.dispatch(ids, 3)
    y = np.stack([ex["E%d" % ids.reshape(-1)[r]]["scale"] * H_[r // 2] + np.array(ex["E%d" % ids.reshape(-1)[r]]["shift"])
                  for r in route_src])
    # pad the width to 8 columns (the library's granularity); extra columns zero
    yp = np.zeros((6, 8), dtype=np.float32)
    yp[:, :2] = y
    out = torch.zeros((3, 8), dtype=torch.float32, device=DEV)
    M.moe_combine(torch.tensor(yp, device=DEV), torch.tensor(gates, device=DEV),
                  torch.tensor(ids, device=DEV), torch.tensor(route_pos, device=DEV), None, out)
    torch.cuda.synchronize()
    assert np.allclose(_np(out)[:, :2], np.array(g["Y"]), atol=1e-6)
    assert np.all(_np(out)[:, 2:] == 0)


# ---------------------------------------------------------------------------
# router and dispatch against the oracle
# ---------------------------------------------------------------------------

ROUTER_CASES = [  # (T, E, K, n_group, topk_group, rsf, norm)
    (257, 8, 2, 1, 1, 1.0, 1),
    (1000, 128, 6, 1, 1, 2.5, 1),
    (1000, 128, 6, 8, 4, 2.5, 1),
    (513, 128, 6, 8, 3, 2.5, 0),
    (300, 512, 22, 1, 1, 1.0, 1),
    (300, 512, 8, 64, 8, 1.5, 1),
    (77, 96, 5, 32, 4, 1.0, 1),
    (64, 1024, 32, 16, 4, 2.0, 1),
    (33, 16, 16, 1, 1, 3.0, 1),
]


@pytest.mark.parametrize("case", ROUTER_CASES, ids=lambda c: "T%d_E%d_K%d_g%d_%d" % c[:5])
def test_route_vs_oracle(case):
    T, E, K, ng, tg, rsf, norm = case
    rng = np.random.default_rng(T * 31 + E)
    z = rng.normal(size=(T, E)).astype(np.float32)
    b = (rng.normal(size=E) * 0.05).astype(np.float32)
    ids, w = M.moe_route(torch.tensor(z, device=DEV), torch.tensor(b, device=DEV), K, ng, tg, norm, rsf)
    torch.cuda.synchronize()
    ids_ref, w_ref, info = O.route(z.astype(np.float64), b, ng, tg, K, norm, rsf)
    bad, near, near_diff = H.compare_ids(_np(ids), ids_ref, info)
    assert len(bad) == 0, (bad[:5], _np(ids)[bad[:3]], ids_ref[bad[:3]])
    ok = np.all(_np(ids) == ids_ref, axis=1)
    assert np.max(np.abs(_np(w)[ok] - w_ref[ok])) <= 1e-6 * rsf
    if norm:
        assert np.allclose(_np(w).sum(1), rsf, rtol=0, atol=1e-6 * rsf)
    print(f"near-tie rows: {len(near)}, of which differing: {len(near_diff)}")


def test_route_exact_ties_lower_id_wins():
    T, E, K = 64, 128, 6
    rng = np.random.default_rng(5)
    z = np.round(rng.normal(size=(T, E)) * 4) / 4  # many bitwise-equal logits
    z = z.astype(np.float32)
    ids, w = M.moe_route(torch.tensor(z, device=DEV), None, K)
    torch.cuda.synchronize()
    ids_ref, _, info = O.route(z.astype(np.float64), None, 1, 1, K, 1, 1.0)
    assert info["exact_tie"].sum() > 10
    assert np.array_equal(_np(ids), ids_ref)


@pytest.mark.parametrize("T,K,E,skew", [(1, 1, 1, False), (1000, 6, 128, False), (4097, 6, 128, True),
                                        (300, 22, 512, False), (2, 2, 3, False), (555, 32, 1024, True)])
def test_dispatch_vs_oracle(T, K, E, skew):
    rng = np.random.default_rng(T + K + E)
    if skew:
        ids = np.stack([np.concatenate([np.arange(K - 1), rng.choice(np.arange(K - 1, E), 1)]) for _ in range(T)])
    else:
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    ids = ids.astype(np.int32)
    counts, offsets, rs, rp = M.moe_dispatch(torch.tensor(ids, device=DEV), E)
    torch.cuda.synchronize()
    c, o, s, p = O.dispatch(ids, E)
    assert np.array_equal(_np(counts), c)
    assert np.array_equal(_np(offsets), o)
    assert np.array_equal(_np(rs), s)
    assert np.array_equal(_np(rp), p)


def test_router_logits_fp32_accuracy():
    """bf16 x against fp32 W_r: the three-plane MFMA product must be as
    accurate as an fp32 dot product (error far below the 1e-5 tie band)."""
    rng = np.random.default_rng(3)
    for (T, d, E) in ((300, 512, 16), (130, 2688, 128), (64, 4096, 512), (5, 264, 24)):
        x = torch.tensor(rng.normal(size=(T, d)).astype(np.float32)).to(torch.bfloat16)
        w = torch.tensor((rng.normal(size=(E, d)) / np.sqrt(d)).astype(np.float32))
        z = M.moe_router_logits(x.to(DEV), w.to(DEV))
        torch.cuda.synchronize()
        ref = O.router_logits(x.to(torch.float64).numpy(), w.numpy())
        err = np.max(np.abs(_np(z) - ref))
        assert err < 2e-6 * np.sqrt(d / 512), (T, d, E, err)


# ---------------------------------------------------------------------------
# the fused layer on small configs (whole-output comparison)
# ---------------------------------------------------------------------------

def _staged(case: H.Case, x=None):
    """The staged calls on the case's inputs (or on ``x``): logits, ids,
    weights, dispatch."""
    cfg = case.cfg
    z = M.moe_router_logits(case.x_dev if x is None else x, case.w_dev["w_router"])
    ids, w = M.moe_route(z, case.w_dev["bias"], cfg.K, cfg.n_group, cfg.topk_group,
                         cfg.norm_topk_prob, cfg.routed_scaling_factor)
    counts, offsets, rs, rp = M.moe_dispatch(ids, cfg.E)
    torch.cuda.synchronize()
    return z, ids, w, counts, offsets, rs, rp


def _check_layer(case: H.Case, flags=0, lazy=False):
    """The fused layer on every row against the oracle (see
    ``_harness.check_layer``): the call's own ids, gates and dispatch, and
    its output by row L2 and per-element error."""
    return H.check_layer(case, flags, lazy=lazy)[0]


def test_tiny_f32_layer():
    case = H.make_case(synth.TINY_F32)
    _check_layer(case)


@pytest.mark.parametrize("kw", [
    dict(),
    dict(T=301, n_group=4, topk_group=2, K=4, name="grouped"),
    dict(T=1, name="one_row"),
    dict(T=129, F_shared=0, name="no_shared"),
    dict(T=200, K=16, name="k_equals_e"),
    dict(T=700, E=8, K=2, F=1024, name="big_chunks"),
    dict(T=150, d=264, F=200, F_shared=136, name="ragged_widths"),
], ids=lambda k: k.get("name", "base"))
def test_small_bf16_layer(kw):
    case = H.make_case(H.small_config(**kw))
    _check_layer(case)


def test_small_f32_layer_grouped():
    case = H.make_case(H.small_config(dtype="f32", T=150, n_group=4, topk_group=2, name="f32g"))
    _check_layer(case)


def test_small_f32_layer_ragged_widths():
    case = H.make_case(H.small_config(dtype="f32", T=70, d=264, F=200, F_shared=136, name="f32r"))
    _check_layer(case)


def test_small_latent_layer():
    cfg = H.small_config(T=200, d=512, d_latent=256, E=32, K=6, F=384, F_shared=512,
                         std_up=256 ** -0.5, std_latent_in=512 ** -0.5, std_latent_out=256 ** -0.5,
                         routed_scaling_factor=1.0, name="latent")
    case = H.make_case(cfg)
    _check_layer(case)


def test_all_rows_to_one_expert():
    """A bias that sends every token to experts 0..K-1: one expert gets all
    T rows (several row chunks), the others none."""
    cfg = H.small_config(T=517, name="hot")
    bias = torch.zeros(cfg.E)
    bias[: cfg.K] = 10.0
    case = H.make_case(cfg, bias=bias)
    _, ids, _, counts, offsets, _, _ = _staged(case)
    assert _np(counts)[: cfg.K].tolist() == [cfg.T] * cfg.K
    _check_layer(case)


def test_zero_skip_layer_and_counts():
    cfg = H.small_config(T=16, name="decode_small")
    case = H.make_case(cfg)
    _check_layer(case, flags=M.MOE_FLAG_ZERO_SKIP_DOWN)
    # staged experts with zero counting: exact zeros of the GPU's own h
    z, ids, w, counts, offsets, rs, rp = _staged(case)
    zc = torch.zeros(2, dtype=torch.int64, device=DEV)
    y1 = M.moe_experts(case.x_dev, cfg.K, rs, offsets, case.w_dev["w_up"], case.w_dev["w_down_t"],
                       flags=M.MOE_FLAG_ZERO_SKIP_DOWN, zero_count=zc)
    y0 = M.moe_experts(case.x_dev, cfg.K, rs, offsets, case.w_dev["w_up"], case.w_dev["w_down_t"])
    torch.cuda.synchronize()
    zeros, skipped = _np(zc).tolist()
    # oracle diagnostic: u in float64, rounded to bf16 like the GPU's epilogue
    x64 = synth.to_f64(case.x_cpu)
    src = _np(rs) // cfg.K
    off = _np(offsets)
    n_zero = 0
    for e in range(cfg.E):
        rows = src[off[e]:off[e + 1]]
        if len(rows) == 0:
            continue
        u = x64[rows] @ case.w_cpu["w_up"][e].to(torch.float64).numpy().T
        ub = torch.tensor(u).to(torch.bfloat16).to(torch.float64).numpy()
        n_zero += int(np.count_nonzero(ub <= 0))
    R = cfg.T * cfg.K
    assert abs(zeros - n_zero) <= max(2, 1e-3 * R * cfg.F), (zeros, n_zero)
    assert 0 <= skipped <= cfg.E * cfg.F
    # the skip path equals the dense path up to fp32 summation order
    a, b = _np(y1.float()), _np(y0.float())
    assert np.max(np.abs(a - b)) <= 1e-2 * np.max(np.abs(b))


def test_fused_equals_staged_bitwise():
    cfg = H.small_config(T=333, name="staged")
    case = H.make_case(cfg)
    y = H.run_fused(case)
    z, ids, w, counts, offsets, rs, rp = _staged(case)
    yr = M.moe_experts(case.x_dev, cfg.K, rs, offsets, case.w_dev["w_up"], case.w_dev["w_down_t"])
    one = torch.tensor([0, cfg.T], dtype=torch.int32, device=DEV)
    ys = M.moe_experts(case.x_dev, 1, None, one, case.w_dev["w_up_shared"][None],
                       case.w_dev["w_down_shared_t"][None])
    # the staged shared expert comes back in the activation dtype; the fused
    # path keeps it in fp32 -- compare the routed part bitwise and the whole
    # output within rounding
    out = torch.empty_like(y)
    M.moe_combine(yr, w, ids, rp, None, out)
    torch.cuda.synchronize()
    y_nos = H.run_fused(H.Case(dataclasses.replace(cfg, F_shared=0), case.w_cpu, case.x_cpu,
                               case.w_dev, case.x_dev))
    assert torch.equal(y_nos, out)
    assert torch.allclose((out.float() + ys.float()), y.float(), rtol=2e-2, atol=2e-2)


def test_determinism_three_runs():
    case = H.make_case(H.small_config(T=999, name="det"))
    ys = [H.run_fused(case).clone() for _ in range(3)]
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[1], ys[2])


def test_accumulate_out():
    case = H.make_case(H.small_config(T=100, name="acc"))
    prev = torch.randn(case.cfg.T, case.cfg.d, device=DEV).to(torch.bfloat16)
    y0 = H.run_fused(case)
    y1 = H.run_fused(case, flags=M.MOE_FLAG_ACCUMULATE_OUT, out=prev.clone())
    diff = (y1.float() - y0.float() - prev.float()).abs().max().item()
    assert diff <= 2e-2 * max(1.0, y1.float().abs().max().item())


def test_zero_rows_is_noop():
    case = H.make_case(H.small_config(T=4, name="z"))
    desc = M.make_desc(case.cfg.params(), M.MOE_BF16)
    out = torch.full((0, case.cfg.d), 7.0, device=DEV).to(torch.bfloat16)
    M.moe_layer_forward(desc, M.make_weights_struct(case.w_dev), case.x_dev[:0], out=out)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# the decode path (MOE_FLAG_ZERO_SKIP_DOWN on bf16 batches of <= 256 rows)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kw", [
    dict(T=1, name="dec_t1"),
    dict(T=3, name="dec_t3"),
    dict(T=64, name="dec_t64"),
    dict(T=256, name="dec_t256"),
    dict(T=257, name="dec_t257_gemm_path"),
    dict(T=40, n_group=4, topk_group=2, K=4, name="dec_grouped"),
    dict(T=33, F_shared=0, name="dec_no_shared"),
    dict(T=20, d=264, F=200, F_shared=136, name="dec_ragged_widths"),
    dict(T=5, d=264, F=200, F_shared=136, name="dec_ragged_widths_small"),
    dict(T=20, K=16, name="dec_k_equals_e"),
    dict(T=48, d=512, d_latent=256, E=32, K=6, F=384, F_shared=512, std_up=256 ** -0.5,
         std_latent_in=512 ** -0.5, std_latent_out=256 ** -0.5, routed_scaling_factor=1.0,
         name="dec_latent"),
    # batches of <= 8 rows with <= 128 experts route and dispatch inside the
    # expert kernel: both edges of that range, grouped routing, every expert
    # touched, 128 experts, a wider expert set that takes the unfused path,
    # no shared expert, and the latent projection
    dict(T=8, name="dec_t8_fused_edge"),
    dict(T=9, name="dec_t9_unfused"),
    dict(T=5, n_group=4, topk_group=2, K=4, name="dec_small_grouped"),
    dict(T=6, K=16, name="dec_small_k_equals_e"),
    dict(T=7, E=128, K=6, F=256, F_shared=0, name="dec_small_e128_no_shared"),
    dict(T=3, E=160, K=6, F=256, name="dec_small_e160_unfused"),
    dict(T=4, d=512, d_latent=256, E=32, K=6, F=384, F_shared=512, std_up=256 ** -0.5,
         std_latent_in=512 ** -0.5, std_latent_out=256 ** -0.5, routed_scaling_factor=1.0,
         name="dec_small_latent"),
], ids=lambda k: k["name"])
def test_decode_path_layer(kw):
    case = H.make_case(H.small_config(**kw))
    _check_layer(case, flags=M.MOE_FLAG_ZERO_SKIP_DOWN)


@pytest.mark.parametrize("T", [24, 5])
def test_decode_path_matches_gemm_path(T):
    """The two paths compute the same layer: outputs agree to bf16 rounding."""
    case = H.make_case(H.small_config(T=T, name="dec_vs_gemm_%d" % T))
    y_dec = H.run_fused(case, flags=M.MOE_FLAG_ZERO_SKIP_DOWN).float()
    y_gemm = H.run_fused(case).float()
    rel = ((y_dec - y_gemm).norm(dim=1) / y_gemm.norm(dim=1)).max().item()
    assert rel <= 1e-2, rel


def test_decode_path_accumulate_and_determinism():
    case = H.make_case(H.small_config(T=16, name="dec_acc"))
    prev = torch.randn(case.cfg.T, case.cfg.d, device=DEV).to(torch.bfloat16)
    f = M.MOE_FLAG_ZERO_SKIP_DOWN
    y0 = H.run_fused(case, flags=f)
    ys = [H.run_fused(case, flags=f | M.MOE_FLAG_ACCUMULATE_OUT, out=prev.clone()) for _ in range(3)]
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[1], ys[2])
    diff = (ys[0].float() - y0.float() - prev.float()).abs().max().item()
    assert diff <= 2e-2 * max(1.0, ys[0].float().abs().max().item())
