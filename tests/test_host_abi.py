"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/moe.h declares, and rejects invalid arguments with the
documented status before launching anything."""
import ctypes
import os
import re

import pytest

import routed_relu_expert_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    return M.lib()


def test_exports_every_declared_function(L):
    names = _declared()
    assert len(names) >= 12, names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(M.EXPORTS)


def test_status_strings(L):
    for st in range(5):
        assert L.moe_status_string(st).decode().startswith("MOE_")


ST = dict(ok=0, inv=1, unsup=2, ws=3)
DUMMY = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


@pytest.mark.parametrize("args,want", [
    # (T, E, K, n_group, topk_group)
    ((4, 8, 9, 1, 1), "inv"),      # K > E
    ((4, 8, 2, 3, 1), "inv"),      # E % n_group
    ((4, 8, 2, 2, 3), "inv"),      # topk_group > n_group
    ((4, 8, 2, 8, 1), "inv"),      # E / n_group < 2
    ((4, 16, 5, 4, 1), "inv"),     # K > topk_group * E / n_group
    ((4, 8, 0, 1, 1), "inv"),      # K < 1
    ((-1, 8, 2, 1, 1), "inv"),     # T < 0
    ((4, 2048, 2, 1, 1), "unsup"), # E > MOE_MAX_EXPERTS
    ((4, 128, 33, 1, 1), "unsup"), # K > MOE_MAX_TOPK
    ((4, 256, 2, 128, 2), "unsup"),  # n_group > MOE_MAX_GROUPS
])
def test_route_rejects(L, args, want):
    T, E, K, ng, tg = args
    st = L.moe_route(DUMMY, None, T, E, K, ng, tg, 1, 1.0, DUMMY, DUMMY, None)
    assert st == ST[want]


def test_route_null_pointers(L):
    assert L.moe_route(None, None, 4, 8, 2, 1, 1, 1, 1.0, DUMMY, DUMMY, None) == ST["inv"]
    assert L.moe_route(DUMMY, None, 4, 8, 2, 1, 1, 1, 1.0, None, DUMMY, None) == ST["inv"]


def test_route_zero_rows_is_ok(L):
    assert L.moe_route(DUMMY, None, 0, 8, 2, 1, 1, 1, 1.0, DUMMY, DUMMY, None) == ST["ok"]


def test_dispatch_rejects(L):
    assert L.moe_dispatch(DUMMY, 4, 3, 2, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 1 << 20, None) == ST["inv"]
    assert L.moe_dispatch(DUMMY, 4, 2, 8, DUMMY, DUMMY, DUMMY, DUMMY, None, 0, None) == ST["ws"]
    assert L.moe_dispatch(DUMMY, 0, 2, 8, DUMMY, DUMMY, DUMMY, DUMMY, None, 0, None) == ST["ok"]


def test_experts_rejects(L):
    # route_src NULL needs K == 1
    assert L.moe_experts(DUMMY, 1, 4, 64, 2, None, DUMMY, 4, 64, DUMMY, DUMMY, 0, DUMMY, None,
                         DUMMY, 1 << 30, None) == ST["inv"]
    # widths not multiples of 8
    assert L.moe_experts(DUMMY, 1, 4, 60, 1, None, DUMMY, 4, 64, DUMMY, DUMMY, 0, DUMMY, None,
                         DUMMY, 1 << 30, None) == ST["unsup"]
    # misaligned pointer
    assert L.moe_experts(ctypes.c_void_p(0x1002), 1, 4, 64, 1, None, DUMMY, 4, 64, DUMMY, DUMMY, 0,
                         DUMMY, None, DUMMY, 1 << 30, None) == ST["unsup"]
    # too small a workspace
    assert L.moe_experts(DUMMY, 1, 4, 64, 1, None, DUMMY, 4, 64, DUMMY, DUMMY, 0, DUMMY, None,
                         DUMMY, 16, None) == ST["ws"]


def test_combine_rejects(L):
    assert L.moe_combine(DUMMY, DUMMY, DUMMY, DUMMY, None, 4, 2, 12, 1, 0, DUMMY, None) == ST["unsup"]
    assert L.moe_combine(None, DUMMY, DUMMY, DUMMY, None, 4, 2, 16, 1, 0, DUMMY, None) == ST["inv"]


def _desc(flags=0, dt=M.MOE_BF16, **kw):
    p = dict(d=256, E=8, K=2, F=512, F_shared=512, n_group=1, topk_group=1,
             routed_scaling_factor=1.0)
    p.update(kw)
    return M.make_desc(p, dt, flags)


def test_layer_forward_rejects(L):
    w = M.LayerWeights(0x1000, 0, 0x1000, 0x1000, 0x1000, 0x1000, 0, 0)
    d = _desc()
    need = L.moe_workspace_size(ctypes.byref(d), 64)
    assert need > 0
    # workspace too small
    assert L.moe_layer_forward(ctypes.byref(d), ctypes.byref(w), DUMMY, 64, DUMMY, DUMMY, need - 1,
                               None) == ST["ws"]
    # missing shared weights
    w2 = M.LayerWeights(0x1000, 0, 0x1000, 0x1000, 0, 0, 0, 0)
    assert L.moe_layer_forward(ctypes.byref(d), ctypes.byref(w2), DUMMY, 64, DUMMY, DUMMY, need,
                               None) == ST["inv"]
    # latent without its projections
    d3 = _desc(d_latent=128)
    assert L.moe_layer_forward(ctypes.byref(d3), ctypes.byref(w), DUMMY, 64, DUMMY, DUMMY, 1 << 40,
                               None) == ST["inv"]
    # unknown flag, bad width
    assert L.moe_layer_forward(ctypes.byref(_desc(flags=64)), ctypes.byref(w), DUMMY, 64, DUMMY,
                               DUMMY, 1 << 40, None) == ST["inv"]
    # MXFP8 activations need MXFP4 experts
    assert L.moe_layer_forward(ctypes.byref(_desc(flags=M.MOE_FLAG_MXFP8_ACTIVATIONS)), ctypes.byref(w), DUMMY, 64,
                               DUMMY, DUMMY, 1 << 40, None) == ST["inv"]
    assert L.moe_layer_forward(ctypes.byref(_desc(d=260)), ctypes.byref(w), DUMMY, 64, DUMMY,
                               DUMMY, 1 << 40, None) == ST["unsup"]
    assert L.moe_workspace_size(ctypes.byref(_desc(K=9)), 64) == 0
    # T == 0: nothing to do
    assert L.moe_layer_forward(ctypes.byref(d), ctypes.byref(w), DUMMY, 0, DUMMY, None, 0,
                               None) == ST["ok"]


def test_operand_size_limits(L):
    """Activation matrices the GEMMs address with 32-bit byte offsets must stay
    under 2^32 bytes: past it the call is rejected, not wrapped."""
    w = M.LayerWeights(0x1000, 0, 0x1000, 0x1000, 0x1000, 0x1000, 0, 0)
    nano = dict(d=2688, E=128, K=6, F=1856, F_shared=3712, routed_scaling_factor=2.5)
    # the Nano layer: y_packed [T*K, d] bf16 is the first to reach 2^32 bytes,
    # at 2^32 / (6 * 2688 * 2) = 133152.5 rows (h [T*K, F] would at 192841.5)
    d = _desc(**nano)
    assert L.moe_workspace_size(ctypes.byref(d), 133152) > 0
    assert L.moe_workspace_size(ctypes.byref(d), 133153) == 0
    assert L.moe_layer_forward(ctypes.byref(d), ctypes.byref(w), DUMMY, 133153, DUMMY, DUMMY, 1 << 40,
                               None) == ST["unsup"]
    # h [T*K, F] alone past the limit (narrow model width)
    dh = _desc(d=8, E=128, K=6, F=1856, F_shared=0)
    assert L.moe_workspace_size(ctypes.byref(dh), 192841) > 0
    assert L.moe_workspace_size(ctypes.byref(dh), 192842) == 0
    # x [T, d] bf16 with d = 8192: 262144 rows reach 2^32 bytes
    dx = _desc(d=8192, E=8, K=1, F=8, F_shared=0)
    assert L.moe_workspace_size(ctypes.byref(dx), 262143) > 0
    assert L.moe_workspace_size(ctypes.byref(dx), 262144) == 0
    # with a shared expert its fp32 rows [T, d] count too: 131072 rows
    dxs = _desc(d=8192, E=8, K=1, F=8, F_shared=8)
    assert L.moe_workspace_size(ctypes.byref(dxs), 131071) > 0
    assert L.moe_workspace_size(ctypes.byref(dxs), 131072) == 0
    # a weight matrix past 2^31 bytes
    assert L.moe_workspace_size(ctypes.byref(_desc(d=8192, E=8, K=1, F=131080, F_shared=0)), 4) == 0
    # the staged experts: h [R, F]
    st = L.moe_experts(DUMMY, 1, 192842, 8, 6, DUMMY, DUMMY, 128, 1856, DUMMY, DUMMY, 0, DUMMY, None,
                       DUMMY, 1 << 40, None)
    assert st == ST["unsup"]
    st = L.moe_experts(DUMMY, 1, 192841, 8, 6, DUMMY, DUMMY, 128, 1856, DUMMY, DUMMY, 0, DUMMY, None,
                       DUMMY, 16, None)
    assert st == ST["ws"]  # within the limits: only the workspace is short
    # the combine: y_packed [T*K, d]
    assert L.moe_combine(DUMMY, DUMMY, DUMMY, DUMMY, None, 131072, 2, 8192, 1, 0, DUMMY, None) == ST["unsup"]
    assert L.moe_combine(DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 131072, 1, 8192, 1, 0, DUMMY, None) == ST["unsup"]


def test_decode_chunk_limit_falls_back(L):
    """The decode path numbers a work item's 64-neuron chunk in 12 bits: a
    hidden width past 4096 chunks takes the grouped GEMMs (the same
    workspace as without the decode flag)."""
    for F, decode in ((4096 * 64, True), (4096 * 64 + 64, False)):
        plain = _desc(d=64, E=8, K=2, F=F, F_shared=0)
        skip = _desc(d=64, E=8, K=2, F=F, F_shared=0, flags=M.MOE_FLAG_ZERO_SKIP_DOWN)
        a, b = L.moe_workspace_size(ctypes.byref(plain), 4), L.moe_workspace_size(ctypes.byref(skip), 4)
        assert a > 0 and b > 0
        assert (a != b) == decode, (F, a, b)


def test_quantize_mxfp8_rejects(L):
    assert L.moe_quantize_mxfp8(DUMMY, 0, 4, 64, DUMMY, DUMMY, 4, None) == ST["inv"]    # fp32 input
    assert L.moe_quantize_mxfp8(DUMMY, 1, 4, 48, DUMMY, DUMMY, 4, None) == ST["unsup"]  # C % 32
    assert L.moe_quantize_mxfp8(DUMMY, 1, 4, 64, DUMMY, DUMMY, 3, None) == ST["inv"]    # ld < rows
    assert L.moe_quantize_mxfp8(None, 1, 4, 64, DUMMY, DUMMY, 4, None) == ST["inv"]
    assert L.moe_quantize_mxfp8(DUMMY, 1, 0, 64, None, None, 0, None) == ST["ok"]
    # the W4A8 layer: with MXFP4 experts, widths multiples of 32, no decode path
    w = M.LayerWeights(0x1000, 0, 0x1000, 0x1000, 0x1000, 0x1000, 0, 0)
    fl = M.MOE_FLAG_MXFP4_EXPERTS | M.MOE_FLAG_MXFP8_ACTIVATIONS
    d = _desc(flags=fl)
    assert L.moe_workspace_size(ctypes.byref(d), 64) > 0
    assert L.moe_workspace_size(ctypes.byref(_desc(flags=fl, d=264)), 64) == 0
    a = L.moe_workspace_size(ctypes.byref(_desc(flags=fl | M.MOE_FLAG_ZERO_SKIP_DOWN)), 4)
    b = L.moe_workspace_size(ctypes.byref(_desc(flags=fl)), 4)
    assert a == b  # the decode flag is a hint the W4A8 layer does not take


def test_workspace_routing_layout(L):
    """The routing offsets lie inside the workspace, do not overlap, and are
    the same whatever path the flags select."""
    for kw, T in ((dict(), 64), (dict(flags=M.MOE_FLAG_ZERO_SKIP_DOWN), 4), (dict(flags=M.MOE_FLAG_ZERO_SKIP_DOWN), 64),
                  (dict(capacity_factor=1.0), 64)):
        d = _desc(**kw)
        lay = M.moe_workspace_routing(d, T)
        need = L.moe_workspace_size(ctypes.byref(d), T)
        K, E = d.K, d.E
        spans = sorted([(lay["ids"], 4 * T * K), (lay["weights"], 4 * T * K), (lay["counts"], 4 * E),
                        (lay["offsets"], 4 * (E + 1)), (lay["route_src"], 4 * T * K), (lay["route_pos"], 4 * T * K)])
        for (a, n), (b, _) in zip(spans, spans[1:]):
            assert a + n <= b
        assert spans[-1][0] + spans[-1][1] <= need
    with pytest.raises(M.MoeError):
        M.moe_workspace_routing(_desc(K=9), 4)


def test_workspace_sizes_grow_with_rows(L):
    d = _desc(d=2688, E=128, K=6, F=1856, F_shared=3712, routed_scaling_factor=2.5)
    a = L.moe_workspace_size(ctypes.byref(d), 64)
    b = L.moe_workspace_size(ctypes.byref(d), 4096)
    assert 0 < a < b
    assert b < 400 * 2 ** 20  # the nano prefill layer needs a few hundred MB


def test_zero_rows_accepts_null_row_pointers(L):
    """T == 0 reads no row pointer: empty tensors hand over NULL."""
    w = M.LayerWeights(0x1000, 0, 0x1000, 0x1000, 0x1000, 0x1000, 0, 0)
    d = _desc()
    assert L.moe_layer_forward(ctypes.byref(d), ctypes.byref(w), None, 0, None, None, 0, None) == ST["ok"]
    assert L.moe_route(None, None, 0, 8, 2, 1, 1, 1, 1.0, None, None, None) == ST["ok"]
    assert L.moe_dispatch(None, 0, 2, 8, None, None, None, None, None, 0, None) == ST["ok"]
    assert L.moe_combine(None, None, None, None, None, 0, 2, 16, 1, 0, None, None) == ST["ok"]
    assert L.moe_experts(None, 1, 0, 64, 2, None, None, 4, 64, None, None, 0, None, None, None, 0,
                         None) == ST["ok"]
    assert L.moe_router_logits(None, 1, 0, 64, None, 8, None, None, 0, None) == ST["ok"]
    # the layer description is still checked
    assert L.moe_layer_forward(ctypes.byref(_desc(K=9)), ctypes.byref(w), None, 0, None, None, 0,
                               None) == ST["inv"]


@pytest.mark.parametrize("args,want", [
    # (dt, G, R, C, kind, src, dst)
    ((1, -1, 4, 8, 0, DUMMY, ctypes.c_void_p(0x100000)), "inv"),     # G < 0
    ((1, 1, -4, 8, 0, DUMMY, ctypes.c_void_p(0x100000)), "inv"),     # R < 0
    ((1, 1, 4, 8, 2, DUMMY, ctypes.c_void_p(0x100000)), "inv"),      # unknown kind
    ((5, 1, 4, 8, 0, DUMMY, ctypes.c_void_p(0x100000)), "inv"),      # unknown dtype
    ((1, 1, 4, 8, 0, None, ctypes.c_void_p(0x100000)), "inv"),       # NULL src
    ((1, 1, 64, 64, 1, DUMMY, ctypes.c_void_p(0x1010)), "inv"),      # dst overlaps src
    ((1, 1, 4, 12, 0, DUMMY, ctypes.c_void_p(0x100000)), "unsup"),   # C % 8
    ((0, 1, 1 << 16, 1 << 14, 0, DUMMY, ctypes.c_void_p(1 << 40)), "unsup"),  # matrix over 2 GiB
    ((1, 1, 4, 8, 0, ctypes.c_void_p(0x1008), ctypes.c_void_p(0x100000)), "unsup"),  # unaligned
    ((1, 0, 4, 8, 0, None, None), "ok"),                             # nothing to pack
])
def test_pack_weight_rejects(L, args, want):
    dt, G, R, C, kind, src, dst = args
    assert L.moe_pack_weight(src, dt, G, R, C, kind, dst, None) == ST[want]


def test_prenorm_flag_rejects(L):
    w = M.LayerWeights(0x1000, 0, 0x1000, 0x1000, 0x1000, 0x1000, 0, 0, 0)
    d = _desc(flags=M.MOE_FLAG_PRENORM_RESIDUAL)
    d.norm_eps = 1e-5
    # no w_norm
    assert L.moe_layer_forward(ctypes.byref(d), ctypes.byref(w), DUMMY, 64, DUMMY, DUMMY, 1 << 40,
                               None) == ST["inv"]
    # not combinable with accumulation
    d2 = _desc(flags=M.MOE_FLAG_PRENORM_RESIDUAL | M.MOE_FLAG_ACCUMULATE_OUT)
    assert L.moe_workspace_size(ctypes.byref(d2), 64) == 0
    # a negative epsilon
    d3 = _desc(flags=M.MOE_FLAG_PRENORM_RESIDUAL)
    d3.norm_eps = -1.0
    assert L.moe_workspace_size(ctypes.byref(d3), 64) == 0
    # the fused front needs room for the normalised rows
    plain = L.moe_workspace_size(ctypes.byref(_desc()), 64)
    assert L.moe_workspace_size(ctypes.byref(d), 64) >= plain + 64 * 256 * 2


@pytest.mark.parametrize("args,want", [
    # (x, w, eps, T, d, dt, out)
    ((DUMMY, DUMMY, 1e-5, -1, 64, 1, DUMMY), "inv"),
    ((DUMMY, DUMMY, -1.0, 4, 64, 1, DUMMY), "inv"),
    ((DUMMY, DUMMY, float("inf"), 4, 64, 1, DUMMY), "inv"),
    ((None, DUMMY, 1e-5, 4, 64, 1, DUMMY), "inv"),
    ((DUMMY, DUMMY, 1e-5, 4, 60, 1, DUMMY), "unsup"),
    ((DUMMY, DUMMY, 1e-5, 4, 16384, 1, DUMMY), "unsup"),
    ((ctypes.c_void_p(0x1008), DUMMY, 1e-5, 4, 64, 1, DUMMY), "unsup"),
    ((None, None, 1e-5, 0, 64, 1, None), "ok"),
])
def test_rmsnorm_rejects(L, args, want):
    assert L.moe_rmsnorm(*args, None) == ST[want]


def test_capacity_rejects(L):
    assert L.moe_capacity_slots(8, 2, 4, 1.25) == 5
    assert L.moe_capacity_slots(8, 2, 4, -1.0) == -1
    assert L.moe_capacity_slots(8, 0, 4, 1.0) == -1
    assert L.moe_capacity_slots(1 << 20, 32, 1, 1e6) == -1  # C past INT_MAX
    ws = L.moe_dispatch_capacity_workspace_size(64, 2, 8)
    assert ws > L.moe_dispatch_workspace_size(64, 2, 8)
    args = [DUMMY, DUMMY, 64, 2, 8, 3, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, ws, None]
    bad = list(args); bad[5] = -1
    assert L.moe_dispatch_capacity(*bad) == ST["inv"]          # negative capacity
    bad = list(args); bad[1] = None
    assert L.moe_dispatch_capacity(*bad) == ST["inv"]          # no gates
    bad = list(args); bad[11] = 16
    assert L.moe_dispatch_capacity(*bad) == ST["ws"]
    zero = [None, None, 0, 2, 8, 3, None, None, None, None, None, 0, None]
    assert L.moe_dispatch_capacity(*zero) == ST["ok"]
    d = _desc()
    d.capacity_factor = -0.5
    assert L.moe_workspace_size(ctypes.byref(d), 64) == 0
    d.capacity_factor = float("inf")
    assert L.moe_workspace_size(ctypes.byref(d), 64) == 0
    d.capacity_factor = 1.0
    assert L.moe_workspace_size(ctypes.byref(d), 64) > L.moe_workspace_size(ctypes.byref(_desc()), 64)


def test_fp8_rejects(L):
    f8 = M.MOE_FLAG_FP8_EXPERTS
    # the quantiser: sizes, dtype, pointers; no rows is a no-op
    assert L.moe_quantize_fp8(DUMMY, 1, -1, 16, DUMMY, DUMMY, None) == ST["inv"]
    assert L.moe_quantize_fp8(DUMMY, 1, 4, 0, DUMMY, DUMMY, None) == ST["inv"]
    assert L.moe_quantize_fp8(DUMMY, M.MOE_FP8_E4M3, 4, 16, DUMMY, DUMMY, None) == ST["inv"]
    assert L.moe_quantize_fp8(DUMMY, 1, 4, 16, DUMMY, None, None) == ST["inv"]
    assert L.moe_quantize_fp8(None, 1, 0, 16, None, None, None) == ST["ok"]
    # one-byte packing needs whole 16-byte column chunks
    assert L.moe_pack_weight(DUMMY, M.MOE_FP8_E4M3, 1, 4, 24, 0, ctypes.c_void_p(0x100000), None) == ST["unsup"]
    assert L.moe_pack_weight(None, M.MOE_FP8_E4M3, 0, 4, 32, 0, None, None) == ST["ok"]
    # the layer: bf16 activations only, widths multiples of 16, scales given
    assert L.moe_workspace_size(ctypes.byref(_desc(flags=f8, dt=M.MOE_F32)), 64) == 0
    assert L.moe_workspace_size(ctypes.byref(_desc(flags=f8, d=264)), 64) == 0
    assert L.moe_workspace_size(ctypes.byref(_desc(flags=f8, F=520)), 64) == 0
    assert L.moe_workspace_size(ctypes.byref(_desc(flags=f8)), 64) > 0
    w = M.LayerWeights(0x1000, 0, 0x1000, 0x1000, 0x1000, 0x1000, 0, 0, 0)
    assert L.moe_layer_forward(ctypes.byref(_desc(flags=f8)), ctypes.byref(w), DUMMY, 64, DUMMY, DUMMY,
                               1 << 40, None) == ST["inv"]  # no scales
    w.w_up_scale = w.w_down_scale = 0x1000
    assert L.moe_layer_forward(ctypes.byref(_desc(flags=f8)), ctypes.byref(w), DUMMY, 64, DUMMY, DUMMY,
                               1 << 40, None) == ST["inv"]  # no shared scales
    w.w_up_shared_scale = 0x1004
    w.w_down_shared_scale = 0x1000
    assert L.moe_layer_forward(ctypes.byref(_desc(flags=f8)), ctypes.byref(w), DUMMY, 64, DUMMY, DUMMY,
                               1 << 40, None) == ST["unsup"]  # unaligned scales
    # the staged FP8 experts: bf16 only, widths multiples of 16, scales given
    args = [DUMMY, 1, 4, 64, 1, None, DUMMY, 4, 64, DUMMY, DUMMY, DUMMY, DUMMY, 0, DUMMY, None, DUMMY,
            1 << 30, None]
    bad = list(args); bad[1] = M.MOE_F32
    assert L.moe_experts_fp8(*bad) == ST["inv"]
    bad = list(args); bad[10] = None
    assert L.moe_experts_fp8(*bad) == ST["inv"]
    bad = list(args); bad[3] = 72
    assert L.moe_experts_fp8(*bad) == ST["unsup"]
    bad = list(args); bad[17] = 16
    assert L.moe_experts_fp8(*bad) == ST["ws"]


def test_mxfp4_rejects(L):
    f4 = M.MOE_FLAG_MXFP4_EXPERTS
    # the quantiser: sizes, dtype, pointers, 32-column blocks; no rows is a no-op
    assert L.moe_quantize_mxfp4(DUMMY, 1, 1, -1, 32, DUMMY, DUMMY, None) == ST["inv"]
    assert L.moe_quantize_mxfp4(DUMMY, 1, 1, 4, 0, DUMMY, DUMMY, None) == ST["inv"]
    assert L.moe_quantize_mxfp4(DUMMY, M.MOE_MXFP4, 1, 4, 32, DUMMY, DUMMY, None) == ST["inv"]
    assert L.moe_quantize_mxfp4(DUMMY, 1, 1, 4, 32, DUMMY, None, None) == ST["inv"]
    assert L.moe_quantize_mxfp4(DUMMY, 1, 1, 4, 48, DUMMY, DUMMY, None) == ST["unsup"]
    assert L.moe_quantize_mxfp4(None, 1, 0, 4, 32, None, None, None) == ST["ok"]
    # 4-bit packing needs whole 32-column blocks
    assert L.moe_pack_weight(DUMMY, M.MOE_MXFP4, 1, 4, 48, 0, ctypes.c_void_p(0x100000), None) == ST["unsup"]
    assert L.moe_pack_weight(None, M.MOE_MXFP4, 0, 4, 64, 0, None, None) == ST["ok"]
    # the layer: bf16 activations, widths multiples of 32, not with FP8, both down packings and scales
    assert L.moe_workspace_size(ctypes.byref(_desc(flags=f4, dt=M.MOE_F32)), 64) == 0
    assert L.moe_workspace_size(ctypes.byref(_desc(flags=f4, d=272)), 64) == 0
    assert L.moe_workspace_size(ctypes.byref(_desc(flags=f4, F=528)), 64) == 0
    assert L.moe_workspace_size(ctypes.byref(_desc(flags=f4 | M.MOE_FLAG_FP8_EXPERTS)), 64) == 0
    assert L.moe_workspace_size(ctypes.byref(_desc(flags=f4)), 64) > 0
    w = M.LayerWeights(0x1000, 0, 0x1000, 0x1000, 0x1000, 0x1000, 0, 0, 0)
    assert L.moe_layer_forward(ctypes.byref(_desc(flags=f4)), ctypes.byref(w), DUMMY, 64, DUMMY, DUMMY,
                               1 << 40, None) == ST["inv"]  # no [OUT_IN] down codes, no scales
    w.w_down = 0x1000
    w.w_up_e8 = w.w_down_e8 = 0x1000
    assert L.moe_layer_forward(ctypes.byref(_desc(flags=f4)), ctypes.byref(w), DUMMY, 64, DUMMY, DUMMY,
                               1 << 40, None) == ST["inv"]  # no shared down codes / scales
    w.w_down_shared = 0x1008
    w.w_up_shared_e8 = w.w_down_shared_e8 = 0x1000
    assert L.moe_layer_forward(ctypes.byref(_desc(flags=f4)), ctypes.byref(w), DUMMY, 64, DUMMY, DUMMY,
                               1 << 40, None) == ST["unsup"]  # unaligned shared down codes
    # the staged MXFP4 experts: bf16 only, widths multiples of 32, codes and scales given
    args = [DUMMY, 1, 4, 64, 1, None, DUMMY, 4, 64, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 0, DUMMY, None,
            DUMMY, 1 << 30, None]
    bad = list(args); bad[1] = M.MOE_F32
    assert L.moe_experts_mxfp4(*bad) == ST["inv"]
    bad = list(args); bad[12] = None
    assert L.moe_experts_mxfp4(*bad) == ST["inv"]
    bad = list(args); bad[3] = 80
    assert L.moe_experts_mxfp4(*bad) == ST["unsup"]
    bad = list(args); bad[18] = 16
    assert L.moe_experts_mxfp4(*bad) == ST["ws"]
    # no backward through MXFP4 experts
    assert L.moe_backward_workspace_size(ctypes.byref(_desc(flags=f4)), 64) == 0


def test_backward_rejects(L):
    w = M.LayerWeights(0x1000, 0, 0x1000, 0x1000, 0x1000, 0x1000, 0, 0, 0)
    wb = M.LayerWeightsBwd(0x1000, 0x1000, 0x1000, 0x1000)
    g = M.LayerGrads(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    d = _desc()
    need = L.moe_backward_workspace_size(ctypes.byref(d), 64)
    assert need > L.moe_workspace_size(ctypes.byref(d), 64)
    # outside the backward's scope
    assert L.moe_backward_workspace_size(ctypes.byref(_desc(dt=M.MOE_F32)), 64) == 0
    assert L.moe_backward_workspace_size(ctypes.byref(_desc(flags=M.MOE_FLAG_FP8_EXPERTS)), 64) == 0
    # a latent layer: its workspace holds the latent rows and their gradients;
    # its projections' packed weights and their gradients are required
    dl = _desc(d_latent=128)
    need_l = L.moe_backward_workspace_size(ctypes.byref(dl), 64)
    assert need_l > 0
    wl = M.LayerWeights(0x1000, 0, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0)
    wbl = M.LayerWeightsBwd(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    gl = M.LayerGrads(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0, 0x1000, 0x1000)
    for bad_wb, bad_g in ((M.LayerWeightsBwd(0x1000, 0x1000, 0x1000, 0x1000, 0, 0x1000), gl),
                          (M.LayerWeightsBwd(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0), gl),
                          (wbl, M.LayerGrads(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0, 0, 0x1000)),
                          (wbl, M.LayerGrads(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0, 0x1000, 0))):
        assert L.moe_layer_backward(ctypes.byref(dl), ctypes.byref(wl), ctypes.byref(bad_wb), DUMMY, DUMMY, 64,
                                    ctypes.byref(bad_g), DUMMY, need_l, None) == ST["inv"]
    # a misaligned latent gradient
    gm = M.LayerGrads(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0, 0x1004, 0x1000)
    assert L.moe_layer_backward(ctypes.byref(dl), ctypes.byref(wl), ctypes.byref(wbl), DUMMY, DUMMY, 64,
                                ctypes.byref(gm), DUMMY, need_l, None) == ST["unsup"]
    assert L.moe_layer_backward(ctypes.byref(_desc(flags=M.MOE_FLAG_ACCUMULATE_OUT)), ctypes.byref(w),
                                ctypes.byref(wb), DUMMY, DUMMY, 64, ctypes.byref(g), DUMMY, need, None) == ST["unsup"]
    # missing backward weights or gradients
    wb2 = M.LayerWeightsBwd(0x1000, 0, 0x1000, 0x1000)
    assert L.moe_layer_backward(ctypes.byref(d), ctypes.byref(w), ctypes.byref(wb2), DUMMY, DUMMY, 64,
                                ctypes.byref(g), DUMMY, need, None) == ST["inv"]
    g2 = M.LayerGrads(0x1000, 0x1000, 0, 0x1000, 0x1000, 0x1000)
    assert L.moe_layer_backward(ctypes.byref(d), ctypes.byref(w), ctypes.byref(wb), DUMMY, DUMMY, 64,
                                ctypes.byref(g2), DUMMY, need, None) == ST["inv"]
    # workspace too small; no rows
    assert L.moe_layer_backward(ctypes.byref(d), ctypes.byref(w), ctypes.byref(wb), DUMMY, DUMMY, 64,
                                ctypes.byref(g), DUMMY, need - 1, None) == ST["ws"]
    assert L.moe_layer_backward(ctypes.byref(d), ctypes.byref(w), ctypes.byref(wb), None, None, 0,
                                ctypes.byref(g), None, 0, None) == ST["ok"]


def test_backward_fused_front_rejects(L):
    """The fused front's backward: in scope, with the norm weight and its
    gradient required."""
    pre = M.MOE_FLAG_PRENORM_RESIDUAL
    d = _desc(flags=pre, norm_eps=1e-5)
    need = L.moe_backward_workspace_size(ctypes.byref(d), 64)
    assert need > L.moe_backward_workspace_size(ctypes.byref(_desc()), 64)  # the normed rows and their gradient
    w = M.LayerWeights(0x1000, 0, 0x1000, 0x1000, 0x1000, 0x1000, 0, 0, 0x1000)
    wb = M.LayerWeightsBwd(0x1000, 0x1000, 0x1000, 0x1000)
    g = M.LayerGrads(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    no_norm = M.LayerWeights(0x1000, 0, 0x1000, 0x1000, 0x1000, 0x1000, 0, 0, 0)
    assert L.moe_layer_backward(ctypes.byref(d), ctypes.byref(no_norm), ctypes.byref(wb), DUMMY, DUMMY, 64,
                                ctypes.byref(g), DUMMY, need, None) == ST["inv"]
    no_dw = M.LayerGrads(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0)
    assert L.moe_layer_backward(ctypes.byref(d), ctypes.byref(w), ctypes.byref(wb), DUMMY, DUMMY, 64,
                                ctypes.byref(no_dw), DUMMY, need, None) == ST["inv"]
    assert L.moe_layer_forward_train(ctypes.byref(d), ctypes.byref(no_norm), DUMMY, 64, DUMMY, DUMMY, need,
                                     None) == ST["inv"]
    assert L.moe_layer_backward(ctypes.byref(d), ctypes.byref(w), ctypes.byref(wb), DUMMY, DUMMY, 64,
                                ctypes.byref(g), DUMMY, need - 1, None) == ST["ws"]
