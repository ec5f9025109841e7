"""The capacity-bounded variant on the GPU through the C ABI: the staged
arbitration bit-exact against the oracle on identical gates (ties
included), and the fused layer against the oracle ("M6.1 - Routed
Capacity", 0x06, 0x06A, 0x05E, 0x05F)."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
import routed_relu_expert_amd as M

from . import _harness as H

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("T,E,K,cf,levels", [
    (64, 8, 2, 1.0, 0), (300, 16, 4, 0.5, 0), (300, 16, 4, 1.25, 8), (1000, 8, 2, 0.25, 4),
    (513, 32, 6, 0.75, 0), (40, 4, 1, 0.0, 3), (2000, 16, 2, 0.1, 0), (7, 8, 8, 1.0, 2)])
def test_capacity_dispatch_matches_oracle(T, E, K, cf, levels):
    rng = np.random.default_rng(T * 31 + E * 7 + K)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    g = rng.random((T, K)).astype(np.float32)
    if levels:  # few distinct gates: the token / slot order decides many ranks
        g = (np.floor(g * levels) / levels).astype(np.float32)
    C = O.capacity_slots(T, K, E, cf) if cf else 0
    assert M.moe_capacity_slots(T, K, E, cf) == (C if cf else 0)
    counts, offsets, src, pos = M.moe_dispatch_capacity(torch.from_numpy(ids).to(DEV),
                                                        torch.from_numpy(g).to(DEV), E, C)
    torch.cuda.synchronize()
    acc, _ = O.arbitrate_capacity(ids, g.astype(np.float64), C)
    c, o, s, p = O.dispatch_accepted(ids, acc, E)
    assert _np(counts).tolist() == c.tolist()
    assert _np(offsets).tolist() == o.tolist()
    assert np.array_equal(_np(src)[:o[-1]], s)
    assert np.array_equal(_np(pos), p)


@pytest.mark.parametrize("T", [8192, 20000])
def test_capacity_hot_expert_radix_select(T):
    """One expert takes a route from every token (thousands of candidates for
    a few slots), with many equal gates.  Past 16384 candidates the kernel
    reads the expert's keys from memory on every pass instead of holding
    them in registers (T = 20000)."""
    E, K = 16, 2
    rng = np.random.default_rng(5)
    ids = np.stack([np.array([0, 1 + rng.integers(0, E - 1)]) for _ in range(T)]).astype(np.int32)
    g = (np.floor(rng.random((T, K)) * 64) / 64).astype(np.float32)
    for C in (1, 100, 4095, T // 2 + 1, T - 1, T):
        counts, offsets, src, pos = M.moe_dispatch_capacity(torch.from_numpy(ids).to(DEV),
                                                            torch.from_numpy(g).to(DEV), E, C)
        acc, _ = O.arbitrate_capacity(ids, g.astype(np.float64), C)
        c, o, s, p = O.dispatch_accepted(ids, acc, E)
        assert _np(counts).tolist() == c.tolist() and _np(offsets).tolist() == o.tolist()
        assert np.array_equal(_np(src)[:o[-1]], s) and np.array_equal(_np(pos), p)


def _check_capacity_layer(case, flags=0, min_gap=1e-6):
    """The capacity-bounded layer on every row (``_harness.check_layer``: the
    fused call's own ids, gates, accepted dispatch and route map against the
    oracle's, outputs by row L2 and per element), on a case whose
    arbitration has no near tie (fp32 gates on the GPU, fp64 in the oracle)
    and that drops routes."""
    cfg = case.cfg
    p = cfg.params()
    ref = O.layer_forward(p, H.synth.to_f64(case.x_cpu), H.oracle_weights(case.w_cpu))
    C = O.capacity_slots(cfg.T, cfg.K, cfg.E, cfg.capacity_factor)
    acc_ref, gap = O.arbitrate_capacity(ref["ids"], ref["weights"], C)
    assert np.all(gap >= min_gap), "choose a case without near-tie arbitration"
    assert (~acc_ref).sum() > 0 or cfg.capacity_factor >= 4, "the case should drop routes"
    y, rt, _ = H.check_layer(case, flags)
    assert np.array_equal(rt["route_pos"] < 0, ~acc_ref.reshape(-1))
    print(f"{cfg.name}: C={C}, dropped {(~acc_ref).sum()} of {acc_ref.size}")


@pytest.mark.parametrize("kw,flags", [
    (dict(T=300, capacity_factor=0.5, name="cap_half"), 0),
    (dict(T=301, capacity_factor=1.0, n_group=4, topk_group=2, name="cap_grouped"), 0),
    (dict(T=200, capacity_factor=0.25, F_shared=0, name="cap_no_shared"), 0),
    (dict(T=64, capacity_factor=0.5, name="cap_decode_flag_falls_back"), M.MOE_FLAG_ZERO_SKIP_DOWN),
    (dict(T=200, d=512, d_latent=256, E=32, K=6, F=384, F_shared=512, std_up=256 ** -0.5,
          std_latent_in=512 ** -0.5, std_latent_out=256 ** -0.5, routed_scaling_factor=1.0,
          capacity_factor=0.5, name="cap_latent"), 0),
    (dict(T=150, dtype="f32", capacity_factor=0.5, name="cap_f32"), 0),
    (dict(T=120, capacity_factor=0.75, prenorm=True, name="cap_prenorm"), 0),
    (dict(T=100, capacity_factor=8.0, name="cap_no_drop"), 0),
], ids=lambda v: v["name"] if isinstance(v, dict) else str(v))
def test_capacity_layer(kw, flags):
    _check_capacity_layer(H.make_case(H.small_config(**kw)), flags)


def test_capacity_deterministic():
    case = H.make_case(H.small_config(T=256, capacity_factor=0.5, name="cap_det"))
    ys = [H.run_fused(case) for _ in range(3)]
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[1], ys[2])
