"""The backward pass on the GPU through the C ABI against the oracle's
gradients ("M6.1 - Routed Capacity", 0x06F steps, taken for the sigmoid
router and ReLU^2 experts): dx, the router, routed-expert and shared-expert
weight gradients, on the plain, grouped, unnormalised, ragged, no-shared and
capacity-bounded layers.  Bar 2e-2: max row-relative error of dx; relative
Frobenius error of each expert's weight gradients, of the router and shared
gradients, and max |error| / max |reference| per tensor; an expert no route
reached has a zero gradient, exactly; repeated calls are bitwise identical."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
import routed_relu_expert_amd as M
from routed_relu_expert_amd import synth

from . import _harness as H

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _glob(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _run(case, wb, dy):
    desc = M.make_desc(case.cfg.params(), M.MOE_BF16)
    g = M.moe_layer_backward(desc, M.make_weights_struct(case.w_dev), wb, case.x_dev, dy)
    torch.cuda.synchronize()
    return g


def _check_backward(kw, seed=5):
    cfg = H.small_config(**kw)
    case = H.make_case(cfg)
    wb = M.device_weights_bwd(case.w_cpu, DEV)
    gen = torch.Generator().manual_seed(seed)
    dy = torch.randn(cfg.T, cfg.d, generator=gen).to(torch.bfloat16)
    g = _run(case, wb, dy.to(DEV))
    p = cfg.params()
    x64 = synth.to_f64(case.x_cpu)
    w64 = H.oracle_weights(case.w_cpu)
    ref = O.layer_backward(p, x64, w64, synth.to_f64(dy))
    info = ref["forward"]["route_info"]
    assert np.all((info["gap"] >= H.NEAR_TIE) | info["exact_tie"]), "choose a case without router near ties"
    # dx rows are sums of many paths: row-relative error.  Weight gradients
    # hold rows that cancel (a dead neuron's row is exactly zero; a gate
    # gradient is a difference of two terms): their error is measured
    # against the size of the gradient, per expert (Frobenius) and per tensor
    # (max |error| / max |reference|).
    errs = {}
    errs["dx"], _ = H.row_error(_np(g["dx"]), ref["dx"])

    def frob(a, b):
        n = np.linalg.norm(b)
        return float(np.linalg.norm(a - b) / n) if n > 0 else float(np.linalg.norm(a))

    got_r = _np(g["dw_router"])
    errs["dw_router"] = frob(got_r, ref["dw_router"])
    errs["dw_router_max"] = _glob(got_r, ref["dw_router"])
    hits = np.diff(np.asarray(ref["forward"]["offsets"]))  # accepted routes per expert
    for k in ("dw_up", "dw_down"):
        got = _np(g[k])
        worst = 0.0
        for e in range(cfg.E):
            if hits[e] == 0:
                assert not got[e].any(), (k, e, "an expert no route reached has zero gradient")
                continue
            worst = max(worst, frob(got[e], ref[k][e]))
        errs[k] = worst
        errs[k + "_max"] = _glob(got, ref[k])
    if cfg.F_shared:
        for k in ("dw_up_shared", "dw_down_shared"):
            errs[k] = frob(_np(g[k]), ref[k])
    print(cfg.name, {k: f"{v:.2e}" for k, v in errs.items()}, "empty experts", int((hits == 0).sum()))
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    return case, wb, dy, g


@pytest.mark.parametrize("kw", [
    dict(T=300, name="bwd_base"),
    dict(T=301, n_group=4, topk_group=2, name="bwd_grouped"),
    dict(T=200, norm_topk_prob=0, routed_scaling_factor=1.0, name="bwd_unnormalised"),
    dict(T=150, d=264, F=200, F_shared=136, std_up=264 ** -0.5, std_down=200 ** -0.5,
         std_up_shared=264 ** -0.5, std_down_shared=136 ** -0.5, name="bwd_ragged"),
    dict(T=129, F_shared=0, name="bwd_no_shared"),
    dict(T=40, E=32, K=2, name="bwd_empty_experts"),
    dict(T=300, capacity_factor=0.5, name="bwd_capacity"),
    dict(T=1, name="bwd_one_row"),
], ids=lambda k: k["name"])
def test_backward_matches_oracle(kw):
    _check_backward(kw)


def test_backward_deterministic():
    case, wb, dy, g = _check_backward(dict(T=257, name="bwd_det"))
    g2 = _run(case, wb, dy.to(DEV))
    for k in g:
        assert torch.equal(g[k], g2[k]), k
