"""The W4A8 expert variant on the GPU through the C ABI: MXFP4 expert
weights and MXFP8 inputs of both expert products on the block-scaled MFMA
(v_mfma_scale_f32_32x32x64_f8f6f4).

* moe_quantize_mxfp8 bit-exact (codes and scales) against the oracle's
  quantiser, on blocks of known outcome (an all-zero block, saturation,
  ties to even in normal and subnormal binades, -0, huge and tiny
  magnitudes) and random rows;
* the fused W4A8 layer against the oracle (which rounds both products'
  inputs through MXFP8 and uses the dequantised MXFP4 weights) on every
  row: grouped, ragged, no shared expert, latent, fused norm front,
  capacity, one row, and the full-size Nano layer;
* repeatable bitwise, and visibly different from the W4A16 layer.
("8 GB Super", "The only number that matters: bytes per token"; "NemotronH",
"How the engine runs it": experts from 4-bit block-scaled checkpoints.)
"""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
import routed_relu_expert_amd as M
from routed_relu_expert_amd import synth

from . import _harness as H

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.detach().cpu().numpy()


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _check_quantizer(xb):
    codes, scales = M.moe_quantize_mxfp8(xb.to(DEV))
    torch.cuda.synchronize()
    ref_c, ref_s = O.quantize_blocks_mxfp8(synth.to_f64(xb))
    assert np.array_equal(_np(scales).T, ref_s), np.argwhere(_np(scales).T != ref_s)[:5]
    bad = np.argwhere(_np(codes) != ref_c)
    assert len(bad) == 0, (bad[:5], _np(codes)[tuple(bad[0])], ref_c[tuple(bad[0])])


def test_quantize_mxfp8_named_blocks():
    x = np.zeros((6, 64), dtype=np.float32)
    x[0, :6] = [256.0, 9.5, 2.0 ** -8 + 2.0 ** -10, 500.0, -3.0, -0.0]    # shared 0: tie, subnormal tie, saturation
    x[0, 32:35] = [1.75 * 2.0 ** 20, 2.0 ** 12 + 2.0 ** 8, -(2.0 ** 20)]   # shared 12
    x[1, :2] = [2.0 ** -130, -(2.0 ** -126)]                            # tiny block (bf16 subnormal amax)
    x[2, :2] = [3.0e38, -1.0]                                            # the largest exponent
    x[3] = np.linspace(-1.0, 1.0, 64)
    x[4, ::2] = 448.0 * 2.0 ** -20                                      # all on one code
    # row 5 stays zero: scale code 0, codes 0
    xb = _bf16(x)
    _check_quantizer(xb)
    codes, scales = M.moe_quantize_mxfp8(xb.to(DEV))
    torch.cuda.synchronize()
    assert _np(scales)[:, 5].tolist() == [0, 0] and not _np(codes)[5].any()
    assert _np(codes)[0, 5] == 0x80  # -0 keeps its sign


@pytest.mark.parametrize("rows,C,seed", [(1, 32, 1), (77, 2688, 2), (300, 1024, 3), (5, 4096, 4)])
def test_quantize_mxfp8_random(rows, C, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, C)).astype(np.float32) * np.exp(rng.uniform(-30, 30, (rows, 1))).astype(np.float32)
    x[:, 7] = 0.0
    _check_quantizer(_bf16(x))


def _w4a8_case(**kw):
    kw.setdefault("expert_dtype", "mxfp4_a8")
    kw.setdefault("d", 512)
    return H.make_case(H.small_config(**kw))


@pytest.mark.parametrize("kw,flags", [
    (dict(T=300, name="w4a8_prefill"), 0),
    (dict(T=301, n_group=4, topk_group=2, name="w4a8_grouped"), 0),
    (dict(T=150, d=288, F=224, F_shared=160, std_up=288 ** -0.5, std_down=224 ** -0.5,
          std_up_shared=288 ** -0.5, std_down_shared=160 ** -0.5, name="w4a8_ragged"), 0),
    (dict(T=129, F_shared=0, name="w4a8_no_shared"), 0),
    (dict(T=200, d=512, d_latent=256, E=32, K=6, F=384, F_shared=512, std_up=256 ** -0.5,
          std_latent_in=512 ** -0.5, std_latent_out=256 ** -0.5, routed_scaling_factor=1.0,
          name="w4a8_latent"), 0),
    (dict(T=120, prenorm=True, name="w4a8_prenorm"), 0),
    (dict(T=1, name="w4a8_one_row"), 0),
    (dict(T=16, name="w4a8_decode_flag_falls_back"), M.MOE_FLAG_ZERO_SKIP_DOWN),
    (dict(T=700, E=8, K=2, F=1024, name="w4a8_big_chunks"), 0),
], ids=lambda v: v["name"] if isinstance(v, dict) else str(v))
def test_w4a8_layer(kw, flags):
    H.check_layer(_w4a8_case(**kw), flags)


def test_w4a8_layer_capacity():
    from .test_gpu_capacity import _check_capacity_layer
    _check_capacity_layer(_w4a8_case(T=300, capacity_factor=0.5, name="w4a8_cap"))


def test_w4a8_deterministic_and_differs_from_w4a16():
    cfg = H.small_config(T=256, d=512, name="w4a8_det")
    c8 = H.make_case(synth.dataclasses.replace(cfg, expert_dtype="mxfp4_a8"))
    ys = [H.run_fused(c8).clone() for _ in range(3)]
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[1], ys[2])
    c16 = H.make_case(synth.dataclasses.replace(cfg, expert_dtype="mxfp4"))
    y16 = H.run_fused(c16).float()
    rel = ((ys[0].float() - y16).norm(dim=1) / y16.norm(dim=1)).max().item()
    assert 1e-3 < rel < 0.2, rel


@pytest.mark.timeout(900)
def test_w4a8_nano_full_size():
    from .test_gpu_full_size import _check_full
    cfg = synth.dataclasses.replace(synth.NANO_PREFILL, expert_dtype="mxfp4_a8", name="nano_w4a8")
    _check_full(H.make_case(cfg))
