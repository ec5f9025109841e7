"""The fused front and back of the layer: RMSNorm in front (within one
rounding of the oracle's float64 norm) and the residual behind, through the C ABI
on the GPU ("NemotronH", "Arithmetic": RMS norm in fp32 times the plain
weight; "M6.1 - Routed Capacity", 0x06F.1: R = H + Y)."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
import routed_relu_expert_amd as M
from routed_relu_expert_amd import synth

from . import _harness as H
from .test_gpu_parity import _check_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,d,eps", [(1, 8, 1e-5), (33, 264, 0.0), (300, 2688, 1e-5), (5, 4096, 1e-2),
                                     (2, 8192, 1e-6), (0, 64, 1e-5), (64, 8192, 1e-5)])
def test_rmsnorm_within_one_rounding(T, d, eps, dtype):
    """moe_rmsnorm against the oracle's float64 definition rounded once.
    bf16: at most one step apart, and a step apart only where the exact value
    lies within the kernel's fp32 error bound of a rounding midpoint.  fp32:
    within that bound (plus the oracle's own half step) of the oracle."""
    rng = np.random.default_rng(T * 7919 + d)
    scale = np.float32(3.0) if d % 3 else np.float32(0.01)
    x = (rng.standard_normal((T, d), dtype=np.float32) * scale)
    w = (np.float32(1.0) + rng.standard_normal(d, dtype=np.float32) * np.float32(0.1))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    xt, wt = torch.from_numpy(x).to(tdt), torch.from_numpy(w).to(tdt)
    y = M.moe_rmsnorm(xt.to(DEV), wt.to(DEV), eps)
    torch.cuda.synchronize()
    v = O.rms_norm_exact(synth.to_f64(xt), synth.to_f64(wt), eps)
    ref = O.round_once(v, dtype)
    got = synth.to_f64(y)
    assert got.shape == ref.shape
    bound = H.rmsnorm_rel_bound(d)
    if dtype == "bf16":
        diff = got != ref
        step = H.bf16_spacing(np.maximum(np.abs(got), np.abs(ref)))
        assert np.all(np.abs(got - ref)[diff] <= step[diff]), np.argwhere(diff)[:5]
        may = H.rmsnorm_may_round_differently(v, d, dtype)
        assert not np.any(diff & ~may), np.argwhere(diff & ~may)[:5]
        print(f"d={d}: {int(diff.sum())} of {diff.size} elements one step from the oracle "
              f"({int(may.sum())} within the bound of a midpoint)")
    else:
        err = np.abs(got - ref)
        assert np.all(err <= (bound + 2 * H.U32) * np.abs(ref) + 1e-45), float(np.max(err / np.maximum(np.abs(ref), 1e-30)))


@pytest.mark.parametrize("kw,flags", [
    (dict(T=300, name="pre_gemm"), 0),
    (dict(T=301, n_group=4, topk_group=2, name="pre_grouped"), 0),
    (dict(T=16, name="pre_decode"), M.MOE_FLAG_ZERO_SKIP_DOWN),
    (dict(T=1, name="pre_decode_t1"), M.MOE_FLAG_ZERO_SKIP_DOWN),
    (dict(T=150, d=264, F=200, F_shared=136, name="pre_ragged"), 0),
    (dict(T=129, F_shared=0, name="pre_no_shared"), 0),
    (dict(T=200, d=512, d_latent=256, E=32, K=6, F=384, F_shared=512, std_up=256 ** -0.5,
          std_latent_in=512 ** -0.5, std_latent_out=256 ** -0.5, routed_scaling_factor=1.0,
          name="pre_latent"), 0),
    (dict(T=48, d=512, d_latent=256, E=32, K=6, F=384, F_shared=512, std_up=256 ** -0.5,
          std_latent_in=512 ** -0.5, std_latent_out=256 ** -0.5, routed_scaling_factor=1.0,
          name="pre_latent_decode"), M.MOE_FLAG_ZERO_SKIP_DOWN),
    (dict(T=70, dtype="f32", name="pre_f32"), 0),
], ids=lambda v: v["name"] if isinstance(v, dict) else str(v))
def test_prenorm_residual_layer(kw, flags):
    case = H.make_case(H.small_config(prenorm=True, **kw))
    _check_layer(case, flags=flags)


def test_prenorm_equals_norm_then_accumulate():
    """The fused layer gives the same bits as RMSNorm, then the layer on its
    output accumulated into an output that holds the hidden state: the
    residual joins the fp32 sum last in both."""
    cfg = H.small_config(prenorm=True, T=200, name="pre_vs_staged")
    case = H.make_case(cfg)
    y_fused = H.run_fused(case)
    xn = M.moe_rmsnorm(case.x_dev, case.w_dev["w_norm"], cfg.norm_eps)
    plain = H.small_config(T=200, name="plain")
    desc = M.make_desc(plain.params(), H.act_code(plain), M.MOE_FLAG_ACCUMULATE_OUT)
    out = case.x_dev.clone()
    M.moe_layer_forward(desc, M.make_weights_struct(case.w_dev), xn, out=out)
    torch.cuda.synchronize()
    assert torch.equal(y_fused, out)


def test_prenorm_deterministic_and_stage_events():
    cfg = H.small_config(prenorm=True, T=64, name="pre_det")
    case = H.make_case(cfg)
    ys = [H.run_fused(case) for _ in range(3)]
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[1], ys[2])
