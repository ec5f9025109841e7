"""moe_layer_forward_noalloc (the entry point for callers that cannot
allocate: its workspace is the library's static device array) against
moe_layer_forward through the C ABI: the same kernels on the same inputs, so
the outputs must be bitwise equal, on two calls in a row with the second on
a smaller input (the array keeps the first call's contents), on the grouped
GEMM path and on the decode path; and a size past the array is rejected."""
import pytest
import torch

import routed_relu_expert_amd as M

from . import _harness as H

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pair(case, flags, T):
    desc = M.make_desc(case.cfg.params(), H.act_code(case.cfg), flags)
    wstruct = M.make_weights_struct(case.w_dev)
    x = case.x_dev[:T]
    y_ref = M.moe_layer_forward(desc, wstruct, x)
    y_na = M.moe_layer_forward_noalloc(desc, wstruct, x)
    torch.cuda.synchronize()
    return y_ref, y_na


@pytest.mark.parametrize("flags,T1,T2", [(0, 300, 37), (M.MOE_FLAG_ZERO_SKIP_DOWN, 16, 3),
                                          (M.MOE_FLAG_ZERO_SKIP_DOWN, 200, 9)],
                         ids=["gemm", "decode", "decode_after_gemm_sized"])
def test_noalloc_matches_forward_twice(flags, T1, T2):
    case = H.make_case(H.small_config(T=T1, name=f"noalloc_{flags}_{T1}"))
    for T in (T1, T2):
        y_ref, y_na = _pair(case, flags, T)
        assert y_na.shape == (T, case.cfg.d)
        assert torch.equal(y_ref, y_na), (T, (y_ref.float() - y_na.float()).abs().max().item())


def test_noalloc_nano_decode_then_smaller():
    """The Nano layer's decode batches: 16 rows, then 1."""
    from routed_relu_expert_amd import synth
    cfg = synth.NANO_DECODE.with_T(16)
    w = synth.make_weights(cfg)
    x = synth.make_inputs(cfg, w)["x"]
    case = H.Case(cfg, w, x, M.device_weights(w, DEV), x.to(DEV))
    for T in (16, 1):
        y_ref, y_na = _pair(case, M.MOE_FLAG_ZERO_SKIP_DOWN, T)
        assert torch.equal(y_ref, y_na), T


def test_noalloc_rejects_past_its_array():
    case = H.make_case(H.small_config(T=8, name="noalloc_big"))
    cfg = case.cfg
    big = dict(cfg.params(), F=1856 * 8, d=2688, E=128, K=6, F_shared=0)
    desc = M.make_desc(big, M.MOE_BF16, 0)
    T = 4096
    assert M.moe_workspace_size(desc, T) > M.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, 2688), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(M.MoeError) as e:
        M.moe_layer_forward_noalloc(desc, M.make_weights_struct(case.w_dev), x)
    assert e.value.status == 2
