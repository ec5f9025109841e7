"""MXFP4 (OCP MX: E2M1 codes, an E8M0 scale per 32 inputs) expert weights on
the GPU through the C ABI: the quantiser bit-exact against the oracle's
(codes and scales), the staged MXFP4 experts and the fused layer against
the oracle's MXFP4 layer (the bf16 layer on the dequantised weights) on the
grouped-GEMM and the decode paths, and sampled rows of the full-size Nano
layer."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
import routed_relu_expert_amd as M
from routed_relu_expert_amd import synth

from . import _harness as H
from .test_gpu_parity import _check_layer, _staged
from .test_gpu_pack import _nibbles

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.detach().cpu().numpy()


def _special_blocks():
    """Blocks with known outcomes: all zero; amax a power of two (lands on 4);
    ties between neighbouring E2M1 values at scale 1 (amax 6); a block that
    saturates (amax / scale = 7); -0."""
    rows = np.zeros((4, 32), np.float32)
    rows[1, 5] = 0.25
    rows[2, :12] = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, -0.0, 0.3, -2.9]
    rows[3, 9] = -0.4375
    rows[3, 10] = 0.2
    return rows


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", [(3, 100, 288), (1, 7, 32), (2, 1, 4096), (1, 1856, 2688)])
def test_quantize_bitexact(shape, dtype):
    g = torch.Generator().manual_seed(sum(shape) + 1)
    w = torch.randn(shape, generator=g) * 0.05
    sp = torch.from_numpy(_special_blocks())
    n = min(4, shape[1])
    w[0, :n, :32] = sp[:n]
    w = w.to(dtype)
    codes, scales = M.moe_quantize_mxfp4(w.to(DEV))
    torch.cuda.synchronize()
    c_ref, s_ref = O.quantize_blocks_mxfp4(w.to(torch.float64).numpy())
    assert codes.shape == shape[:-1] + (shape[-1] // 2,) and scales.shape == (shape[0], shape[-1] // 32, shape[1])
    assert np.array_equal(_np(scales), np.swapaxes(s_ref, -1, -2))
    assert np.array_equal(_nibbles(_np(codes)), c_ref)


def test_quantize_special_block_codes():
    """The special blocks against codes written out from the format's
    definition."""
    codes, scales = M.moe_quantize_mxfp4(torch.from_numpy(_special_blocks()).to(DEV))
    c, sc = _nibbles(_np(codes)), _np(scales)[0]
    # zero block: scale code 0, codes 0; amax 0.25: shared -4 (0.25 / 2^-4 = 4 -> code 6)
    assert sc[0] == 0 and np.all(c[0] == 0)
    assert sc[1] == 127 - 4 and c[1, 5] == 6
    # amax 6: shared 0; 0.25 -> 0, 0.75 -> 1.0 (2), 1.25 -> 1.0 (2), 1.75 -> 2 (4),
    # 2.5 -> 2 (4), 3.5 -> 4 (6), 5 -> 4 (6), -5 -> -4 (14), -0 -> 8, 0.3 -> 0.5 (1), -2.9 -> -3 (13)
    assert sc[2] == 127 and c[2, :12].tolist() == [7, 0, 2, 2, 4, 4, 6, 6, 14, 8, 1, 13]
    # amax 0.4375: shared -4, 7 saturates to 6 (code 15 negative); 0.2 * 16 = 3.2 -> 3 (5)
    assert sc[3] == 127 - 4 and c[3, 9] == 15 and c[3, 10] == 5


def _fp4_case(**kw):
    kw.setdefault("expert_dtype", "mxfp4")
    return H.make_case(H.small_config(**kw))


@pytest.mark.parametrize("T,flags", [(300, 0), (16, M.MOE_FLAG_ZERO_SKIP_DOWN), (3, M.MOE_FLAG_ZERO_SKIP_DOWN)],
                         ids=["gemm", "decode16", "decode3"])
def test_staged_experts_mxfp4(T, flags):
    case = _fp4_case(T=T, name=f"st4_{T}")
    cfg = case.cfg
    z, ids, w, counts, offsets, rs, rp = _staged(case)
    wd = case.w_dev
    y = M.moe_experts_mxfp4(case.x_dev, cfg.K, rs, offsets, wd["w_up"], wd["w_up_e8"], wd["w_down_t"],
                            wd["w_down"], wd["w_down_e8"], flags=flags)
    torch.cuda.synchronize()
    x64 = synth.to_f64(case.x_cpu)
    w4 = O.mxfp4_expert_weights(H.oracle_weights(case.w_cpu))
    src, off = _np(rs) // cfg.K, _np(offsets)
    yg = _np(y.float()).astype(np.float64)
    worst = 0.0
    for e in range(cfg.E):
        if off[e + 1] == off[e]:
            continue
        ref = O.expert_mlp(x64[src[off[e]:off[e + 1]]], w4["w_up"][e], w4["w_down"][e])
        rel, _ = H.row_error(yg[off[e]:off[e + 1]], ref)
        worst = max(worst, rel, float(H.elementwise_row_error(yg[off[e]:off[e + 1]], ref).max()))
    print(f"staged mxfp4 T={T}: max row rel err {worst:.3e}")
    assert worst <= H.TOL["bf16"], worst


@pytest.mark.parametrize("kw,flags", [
    (dict(T=300, name="fp4_prefill"), 0),
    (dict(T=301, n_group=4, topk_group=2, name="fp4_grouped"), 0),
    (dict(T=150, d=288, F=224, F_shared=160, std_up=288 ** -0.5, std_down=224 ** -0.5,
          std_up_shared=288 ** -0.5, std_down_shared=160 ** -0.5, name="fp4_ragged"), 0),
    (dict(T=129, F_shared=0, name="fp4_no_shared"), 0),
    (dict(T=200, d=512, d_latent=256, E=32, K=6, F=384, F_shared=512, std_up=256 ** -0.5,
          std_latent_in=512 ** -0.5, std_latent_out=256 ** -0.5, routed_scaling_factor=1.0,
          name="fp4_latent"), 0),
    (dict(T=120, prenorm=True, name="fp4_prenorm"), 0),
    (dict(T=1, name="fp4_dec_t1"), M.MOE_FLAG_ZERO_SKIP_DOWN),
    (dict(T=4, name="fp4_dec_t4"), M.MOE_FLAG_ZERO_SKIP_DOWN),
    (dict(T=9, name="fp4_dec_t9"), M.MOE_FLAG_ZERO_SKIP_DOWN),
    (dict(T=64, name="fp4_dec_t64"), M.MOE_FLAG_ZERO_SKIP_DOWN),
    (dict(T=20, d=288, F=224, F_shared=160, std_up=288 ** -0.5, std_down=224 ** -0.5,
          std_up_shared=288 ** -0.5, std_down_shared=160 ** -0.5, name="fp4_dec_ragged"),
     M.MOE_FLAG_ZERO_SKIP_DOWN),
    (dict(T=5, d=288, F=224, F_shared=160, std_up=288 ** -0.5, std_down=224 ** -0.5,
          std_up_shared=288 ** -0.5, std_down_shared=160 ** -0.5, name="fp4_dec_ragged_small"),
     M.MOE_FLAG_ZERO_SKIP_DOWN),
    (dict(T=48, d=512, d_latent=256, E=32, K=6, F=384, F_shared=512, std_up=256 ** -0.5,
          std_latent_in=512 ** -0.5, std_latent_out=256 ** -0.5, routed_scaling_factor=1.0,
          name="fp4_dec_latent"), M.MOE_FLAG_ZERO_SKIP_DOWN),
    (dict(T=16, prenorm=True, name="fp4_dec_prenorm"), M.MOE_FLAG_ZERO_SKIP_DOWN),
], ids=lambda v: v["name"] if isinstance(v, dict) else str(v))
def test_mxfp4_layer(kw, flags):
    _check_layer(_fp4_case(**kw), flags=flags)


def test_mxfp4_layer_capacity():
    from .test_gpu_capacity import _check_capacity_layer
    _check_capacity_layer(_fp4_case(T=300, capacity_factor=0.5, name="fp4_cap"))


def test_mxfp4_decode_matches_gemm_and_is_deterministic():
    case = _fp4_case(T=24, name="fp4_dec_vs_gemm")
    f = M.MOE_FLAG_ZERO_SKIP_DOWN
    ys = [H.run_fused(case, flags=f).clone() for _ in range(3)]
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[1], ys[2])
    y_gemm = H.run_fused(case).float()
    rel = ((ys[0].float() - y_gemm).norm(dim=1) / y_gemm.norm(dim=1)).max().item()
    assert rel <= 1e-2, rel


def test_mxfp4_differs_from_bf16_layer():
    """The MXFP4 layer is not the bf16 layer: the quantisation error is seen
    (and stays within what 4-bit elements with block scales allow)."""
    cfg = H.small_config(T=64, name="fp4_vs_bf16")
    c16 = H.make_case(cfg)
    c4 = H.make_case(synth.dataclasses.replace(cfg, expert_dtype="mxfp4"))
    y16, y4 = H.run_fused(c16).float(), H.run_fused(c4).float()
    rel = ((y4 - y16).norm(dim=1) / y16.norm(dim=1)).max().item()
    assert 1e-2 < rel < 0.5, rel


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T,flags", [(4096, 0), (1, M.MOE_FLAG_ZERO_SKIP_DOWN),
                                              (16, M.MOE_FLAG_ZERO_SKIP_DOWN)],
                         ids=["prefill4096", "decode1", "decode16"])
def test_mxfp4_nano_full_size(T, flags):
    from .test_gpu_full_size import _check_full
    cfg = synth.dataclasses.replace(synth.NANO_PREFILL, expert_dtype="mxfp4", name="nano_fp4").with_T(T)
    if T != synth.NANO_PREFILL.T:
        cfg = synth.dataclasses.replace(cfg, x_seed=synth.NANO_DECODE.x_seed)
    _check_full(H.make_case(cfg), flags=flags)
