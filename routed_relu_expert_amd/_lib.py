"""ctypes binding of libmoe (include/moe.h).

Argument marshalling only: every computation runs in the HIP kernels of
libmoe.so.  PyTorch supplies device memory (tensors, workspaces) and the
stream (``torch.cuda.current_stream()``).  The library is loaded on first
use and a missing or unloadable library raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP4 = 0, 1, 2, 3
MOE_FLAG_ZERO_SKIP_DOWN = 1
MOE_FLAG_ACCUMULATE_OUT = 2
MOE_FLAG_PRENORM_RESIDUAL = 4
MOE_FLAG_FP8_EXPERTS = 8
MOE_FLAG_MXFP4_EXPERTS = 16
MOE_FLAG_MXFP8_ACTIVATIONS = 32
MOE_MAX_EXPERTS, MOE_MAX_TOPK, MOE_MAX_GROUPS = 1024, 32, 64
MOE_PACK_OUT_IN, MOE_PACK_NEURON_MAJOR = 0, 1
STAGES = ("router_gemm", "route", "dispatch", "latent_in", "up", "down", "combine", "latent_out", "norm")

EXPORTS = (
    "moe_router_logits_workspace_size", "moe_router_logits", "moe_route",
    "moe_dispatch_workspace_size", "moe_dispatch", "moe_experts_workspace_size",
    "moe_experts", "moe_combine", "moe_workspace_size", "moe_layer_forward",
    "moe_layer_forward_timed", "moe_status_string", "moe_pack_weight", "moe_rmsnorm",
    "moe_capacity_slots", "moe_dispatch_capacity_workspace_size", "moe_dispatch_capacity",
    "moe_quantize_fp8", "moe_experts_fp8", "moe_backward_workspace_size", "moe_layer_backward",
    "moe_layer_backward_timed", "moe_layer_forward_train", "moe_layer_backward_saved",
    "moe_quantize_mxfp4", "moe_experts_mxfp4", "moe_workspace_routing", "moe_layer_forward_noalloc",
    "moe_quantize_mxfp8",
)
BWD_STAGES = ("forward", "gates", "dh", "dx", "transpose", "dw_down", "dw_up")


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_status_string(status)}")


class LayerDesc(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int), ("E", ctypes.c_int), ("K", ctypes.c_int),
                ("F", ctypes.c_int), ("F_shared", ctypes.c_int), ("d_latent", ctypes.c_int),
                ("n_group", ctypes.c_int), ("topk_group", ctypes.c_int),
                ("norm_topk_prob", ctypes.c_int), ("routed_scaling_factor", ctypes.c_float),
                ("act_dtype", ctypes.c_int), ("flags", ctypes.c_int), ("norm_eps", ctypes.c_float),
                ("capacity_factor", ctypes.c_float)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_router", "bias", "w_up", "w_down_t", "w_up_shared", "w_down_shared_t",
        "w_latent_in", "w_latent_out", "w_norm", "w_up_scale", "w_down_scale",
        "w_up_shared_scale", "w_down_shared_scale", "w_down", "w_down_shared", "w_up_e8", "w_down_e8",
        "w_up_shared_e8", "w_down_shared_e8")]


class RoutingLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("ids", "weights", "counts", "offsets", "route_src", "route_pos")]


class LayerWeightsBwd(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_up_nm", "w_down_nm", "w_up_shared_nm", "w_down_shared_nm", "w_latent_in_nm", "w_latent_out_nm")]


class LayerGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "dx", "dw_router", "dw_up", "dw_down", "dw_up_shared", "dw_down_shared", "dw_norm", "dw_latent_in",
        "dw_latent_out")]


_lib = None

P, I, F, Z, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """Load libmoe.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "moe_router_logits_workspace_size": (Z, [I, I, I, I]),
        "moe_router_logits": (I, [P, I, I, I, P, I, P, P, Z, S]),
        "moe_route": (I, [P, P, I, I, I, I, I, I, F, P, P, S]),
        "moe_dispatch_workspace_size": (Z, [I, I, I]),
        "moe_dispatch": (I, [P, I, I, I, P, P, P, P, P, Z, S]),
        "moe_experts_workspace_size": (Z, [I, I, I, I, I, I, I]),
        "moe_experts": (I, [P, I, I, I, I, P, P, I, I, P, P, I, P, P, P, Z, S]),
        "moe_combine": (I, [P, P, P, P, P, I, I, I, I, I, P, S]),
        "moe_workspace_size": (Z, [ctypes.POINTER(LayerDesc), I]),
        "moe_layer_forward": (I, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights),
                                  P, I, P, P, Z, S]),
        "moe_layer_forward_timed": (I, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights),
                                        P, I, P, P, Z, S, P]),
        "moe_status_string": (ctypes.c_char_p, [I]),
        "moe_pack_weight": (I, [P, I, I, I, I, I, P, S]),
        "moe_rmsnorm": (I, [P, P, F, I, I, I, P, S]),
        "moe_capacity_slots": (I, [I, I, I, F]),
        "moe_dispatch_capacity_workspace_size": (Z, [I, I, I]),
        "moe_dispatch_capacity": (I, [P, P, I, I, I, I, P, P, P, P, P, Z, S]),
        "moe_quantize_fp8": (I, [P, I, ctypes.c_long, I, P, P, S]),
        "moe_experts_fp8": (I, [P, I, I, I, I, P, P, I, I, P, P, P, P, I, P, P, P, Z, S]),
        "moe_quantize_mxfp4": (I, [P, I, I, I, I, P, P, S]),
        "moe_quantize_mxfp8": (I, [P, I, I, I, P, P, ctypes.c_long, S]),
        "moe_experts_mxfp4": (I, [P, I, I, I, I, P, P, I, I, P, P, P, P, P, I, P, P, P, Z, S]),
        "moe_backward_workspace_size": (Z, [ctypes.POINTER(LayerDesc), I]),
        "moe_layer_backward": (I, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights),
                                   ctypes.POINTER(LayerWeightsBwd), P, P, I, ctypes.POINTER(LayerGrads),
                                   P, Z, S]),
        "moe_layer_backward_timed": (I, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights),
                                         ctypes.POINTER(LayerWeightsBwd), P, P, I, ctypes.POINTER(LayerGrads),
                                         P, Z, S, P, I]),
        "moe_layer_backward_saved": (I, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights),
                                         ctypes.POINTER(LayerWeightsBwd), P, P, I, ctypes.POINTER(LayerGrads),
                                         P, Z, S]),
        "moe_layer_forward_train": (I, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), P, I, P, P, Z, S]),
        "moe_workspace_routing": (I, [ctypes.POINTER(LayerDesc), I, ctypes.POINTER(RoutingLayout)]),
        "moe_layer_forward_noalloc": (I, [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), P, I, P, S]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _status_string(st: int) -> str:
    return lib().moe_status_string(st).decode()


def _check(st: int, what: str):
    if st != MOE_OK:
        raise MoeError(st, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported activation dtype {t.dtype}")


def _wdt(t: torch.Tensor) -> int:
    """Weight dtype: an activation dtype, or uint8 E4M3 codes."""
    return MOE_FP8_E4M3 if t.dtype == torch.uint8 else _dt(t)


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# staged calls
# ---------------------------------------------------------------------------

def moe_router_logits(x: torch.Tensor, w_router: torch.Tensor, logits=None, ws=None, stream=None):
    T, d = x.shape
    E = w_router.shape[0]
    dt = _dt(x)
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    need = lib().moe_router_logits_workspace_size(T, d, E, dt)
    if ws is None:
        ws = _workspace(need, x.device)
    _check(lib().moe_router_logits(_ptr(x), dt, T, d, _ptr(w_router), E, _ptr(logits), _ptr(ws),
                                   ws.numel(), _stream(stream)), "moe_router_logits")
    return logits


def moe_route(logits: torch.Tensor, bias, K: int, n_group: int = 1, topk_group: int = 1,
              norm_topk_prob: int = 1, routed_scaling_factor: float = 1.0, ids=None, weights=None,
              stream=None):
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, K), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((T, K), dtype=torch.float32, device=logits.device)
    _check(lib().moe_route(_ptr(logits), _ptr(bias), T, E, K, n_group, topk_group,
                           int(norm_topk_prob), float(routed_scaling_factor), _ptr(ids),
                           _ptr(weights), _stream(stream)), "moe_route")
    return ids, weights


def moe_dispatch(ids: torch.Tensor, E: int, stream=None):
    T, K = ids.shape
    dev = ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    route_src = torch.empty(T * K, dtype=torch.int32, device=dev)
    route_pos = torch.empty(T * K, dtype=torch.int32, device=dev)
    ws = _workspace(lib().moe_dispatch_workspace_size(T, K, E), dev)
    _check(lib().moe_dispatch(_ptr(ids), T, K, E, _ptr(counts), _ptr(offsets), _ptr(route_src),
                              _ptr(route_pos), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_dispatch")
    return counts, offsets, route_src, route_pos


def moe_capacity_slots(T: int, K: int, E: int, capacity_factor: float) -> int:
    return int(lib().moe_capacity_slots(T, K, E, float(capacity_factor)))


def moe_dispatch_capacity(ids: torch.Tensor, weights: torch.Tensor, E: int, capacity: int, stream=None):
    """Capacity-bounded dispatch: (counts, offsets, route_src [accepted rows
    first], route_pos with -1 for overflowed routes)."""
    T, K = ids.shape
    dev = ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    route_src = torch.empty(T * K, dtype=torch.int32, device=dev)
    route_pos = torch.empty(T * K, dtype=torch.int32, device=dev)
    ws = _workspace(lib().moe_dispatch_capacity_workspace_size(T, K, E), dev)
    _check(lib().moe_dispatch_capacity(_ptr(ids), _ptr(weights), T, K, E, int(capacity), _ptr(counts),
                                       _ptr(offsets), _ptr(route_src), _ptr(route_pos), _ptr(ws), ws.numel(),
                                       _stream(stream)), "moe_dispatch_capacity")
    return counts, offsets, route_src, route_pos


def moe_experts(x: torch.Tensor, K: int, route_src, offsets: torch.Tensor, w_up: torch.Tensor,
                w_down_t: torch.Tensor, flags: int = 0, y_packed=None, zero_count=None,
                ws=None, stream=None):
    T, d_e = x.shape
    E, F, _ = w_up.shape
    dt = _dt(x)
    if y_packed is None:
        y_packed = torch.empty((T * K, d_e), dtype=x.dtype, device=x.device)
    need = lib().moe_experts_workspace_size(dt, T, d_e, K, E, F, flags)
    if ws is None:
        ws = _workspace(need, x.device)
    _check(lib().moe_experts(_ptr(x), dt, T, d_e, K, _ptr(route_src), _ptr(offsets), E, F,
                             _ptr(w_up), _ptr(w_down_t), flags, _ptr(y_packed), _ptr(zero_count),
                             _ptr(ws), ws.numel(), _stream(stream)), "moe_experts")
    return y_packed


def moe_experts_fp8(x: torch.Tensor, K: int, route_src, offsets: torch.Tensor, w_up: torch.Tensor,
                    w_up_scale: torch.Tensor, w_down_t: torch.Tensor, w_down_scale: torch.Tensor,
                    flags: int = 0, y_packed=None, zero_count=None, ws=None, stream=None):
    """moe_experts with packed E4M3 codes (uint8) and fp32 per-output-channel scales."""
    T, d_e = x.shape
    E, F, _ = w_up.shape
    dt = _dt(x)
    if y_packed is None:
        y_packed = torch.empty((T * K, d_e), dtype=x.dtype, device=x.device)
    need = lib().moe_experts_workspace_size(dt, T, d_e, K, E, F, flags)
    if ws is None:
        ws = _workspace(need, x.device)
    _check(lib().moe_experts_fp8(_ptr(x), dt, T, d_e, K, _ptr(route_src), _ptr(offsets), E, F,
                                 _ptr(w_up), _ptr(w_up_scale), _ptr(w_down_t), _ptr(w_down_scale), flags,
                                 _ptr(y_packed), _ptr(zero_count), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_experts_fp8")
    return y_packed


def moe_experts_mxfp4(x: torch.Tensor, K: int, route_src, offsets: torch.Tensor, w_up: torch.Tensor,
                      w_up_e8: torch.Tensor, w_down_t: torch.Tensor, w_down: torch.Tensor,
                      w_down_e8: torch.Tensor, flags: int = 0, y_packed=None, zero_count=None, ws=None,
                      stream=None):
    """moe_experts with packed MXFP4 codes (uint8, two per byte) and E8M0
    block scales; the down codes in both packings (w_down_t neuron-major,
    w_down [OUT_IN])."""
    T, d_e = x.shape
    E, F = w_up.shape[0], w_up.shape[1]
    dt = _dt(x)
    if y_packed is None:
        y_packed = torch.empty((T * K, d_e), dtype=x.dtype, device=x.device)
    need = lib().moe_experts_workspace_size(dt, T, d_e, K, E, F, flags)
    if ws is None:
        ws = _workspace(need, x.device)
    _check(lib().moe_experts_mxfp4(_ptr(x), dt, T, d_e, K, _ptr(route_src), _ptr(offsets), E, F,
                                   _ptr(w_up), _ptr(w_up_e8), _ptr(w_down_t), _ptr(w_down), _ptr(w_down_e8),
                                   flags, _ptr(y_packed), _ptr(zero_count), _ptr(ws), ws.numel(),
                                   _stream(stream)), "moe_experts_mxfp4")
    return y_packed


def moe_quantize_mxfp8(x: torch.Tensor, stream=None):
    """MXFP8 codes [rows, C] (uint8 E4M3) and block-major E8M0 scales
    [C / 32, rows] of bf16 rows x [rows, C]."""
    x = x.contiguous()
    rows, C = x.shape
    codes = torch.empty((rows, C), dtype=torch.uint8, device=x.device)
    scales = torch.empty((C // 32, rows), dtype=torch.uint8, device=x.device)
    _check(lib().moe_quantize_mxfp8(_ptr(x), _dt(x), rows, C, _ptr(codes), _ptr(scales), rows, _stream(stream)),
           "moe_quantize_mxfp8")
    return codes, scales


def moe_quantize_mxfp4(w: torch.Tensor, stream=None):
    """MXFP4 quantisation of [R, C] or [G, R, C] device weights in [out, in]
    storage, blocks of 32 along C: (codes uint8 [..., R, C / 2], element 2i
    in the low nibble; scales uint8 [..., C / 32, R], block-major)."""
    w = w.contiguous()
    G, R, C = (1, *w.shape) if w.dim() == 2 else w.shape
    codes = torch.empty(w.shape[:-1] + (C // 2,), dtype=torch.uint8, device=w.device)
    scales = torch.empty(w.shape[:-2] + (C // 32, R), dtype=torch.uint8, device=w.device)
    _check(lib().moe_quantize_mxfp4(_ptr(w), _dt(w), G, R, C, _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_quantize_mxfp4")
    return codes, scales


def fp4_transpose(codes: torch.Tensor) -> torch.Tensor:
    """The transpose of [..., R, C] 4-bit codes stored two per byte
    ([..., R, C / 2] uint8, element 2i in the low nibble) in the same
    storage: [..., C, R / 2].  Moves codes only (weight preparation)."""
    n = torch.stack((codes & 15, codes >> 4), dim=-1).flatten(-2)
    nt = n.transpose(-1, -2).contiguous()
    return (nt[..., 0::2] | (nt[..., 1::2] << 4)).contiguous()


def moe_quantize_fp8(w: torch.Tensor, codes=None, scales=None, stream=None):
    """Per-row FP8 (E4M3) quantisation of [..., R, C] device weights in
    [out, in] storage: (codes uint8 [..., R, C], scales fp32 [..., R])."""
    w = w.contiguous()
    C = w.shape[-1]
    rows = w.numel() // C if C else 0
    if codes is None:
        codes = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(w.shape[:-1], dtype=torch.float32, device=w.device)
    _check(lib().moe_quantize_fp8(_ptr(w), _dt(w), rows, C, _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_quantize_fp8")
    return codes, scales


def moe_rmsnorm(x: torch.Tensor, w_norm: torch.Tensor, eps: float, out=None, stream=None):
    T, d = x.shape
    if out is None:
        out = torch.empty_like(x)
    _check(lib().moe_rmsnorm(_ptr(x), _ptr(w_norm), float(eps), T, d, _dt(x), _ptr(out), _stream(stream)),
           "moe_rmsnorm")
    return out


def moe_combine(y_packed, weights, ids, route_pos, y_shared, out, flags: int = 0, stream=None):
    T, K = ids.shape
    d = out.shape[1]
    _check(lib().moe_combine(_ptr(y_packed), _ptr(weights), _ptr(ids), _ptr(route_pos),
                             _ptr(y_shared), T, K, d, _dt(out), flags, _ptr(out), _stream(stream)),
           "moe_combine")
    return out


# ---------------------------------------------------------------------------
# fused layer
# ---------------------------------------------------------------------------

def make_desc(p: dict, act_dtype: int, flags: int = 0) -> LayerDesc:
    if p.get("prenorm_residual"):
        flags |= MOE_FLAG_PRENORM_RESIDUAL
    if p.get("expert_dtype") == "fp8":
        flags |= MOE_FLAG_FP8_EXPERTS
    if p.get("expert_dtype") in ("mxfp4", "mxfp4_a8"):
        flags |= MOE_FLAG_MXFP4_EXPERTS
    if p.get("expert_dtype") == "mxfp4_a8":
        flags |= MOE_FLAG_MXFP8_ACTIVATIONS
    return LayerDesc(p["d"], p["E"], p["K"], p["F"], p.get("F_shared", 0), p.get("d_latent", 0),
                     p["n_group"], p["topk_group"], int(p.get("norm_topk_prob", 1)),
                     float(p["routed_scaling_factor"]), act_dtype, flags, float(p.get("norm_eps", 0.0)),
                     float(p.get("capacity_factor", 0.0)))


def make_weights_struct(w: dict) -> LayerWeights:
    """``w``: device tensors keyed like LayerWeights' fields (w_down_t and
    w_down_shared_t neuron-major); missing keys are NULL."""
    return LayerWeights(*[(w[n].data_ptr() if w.get(n) is not None else None)
                          for n, _ in LayerWeights._fields_])


def moe_workspace_size(desc: LayerDesc, T: int) -> int:
    return lib().moe_workspace_size(ctypes.byref(desc), T)


def moe_layer_forward(desc: LayerDesc, wstruct: LayerWeights, x: torch.Tensor, out=None, ws=None,
                      stream=None, events=None):
    T = x.shape[0]
    if out is None:
        out = torch.empty((T, desc.d), dtype=x.dtype, device=x.device)
    if ws is None:
        ws = _workspace(moe_workspace_size(desc, T), x.device)
    if events is None:
        st = lib().moe_layer_forward(ctypes.byref(desc), ctypes.byref(wstruct), _ptr(x), T,
                                     _ptr(out), _ptr(ws), ws.numel(), _stream(stream))
    else:
        st = lib().moe_layer_forward_timed(ctypes.byref(desc), ctypes.byref(wstruct), _ptr(x), T,
                                           _ptr(out), _ptr(ws), ws.numel(), _stream(stream),
                                           events)
    _check(st, "moe_layer_forward")
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES


def moe_layer_forward_noalloc(desc: LayerDesc, wstruct: LayerWeights, x: torch.Tensor, out=None, stream=None):
    """moe_layer_forward with the library's own static workspace (no
    workspace argument; the call allocates nothing)."""
    T = x.shape[0]
    if out is None:
        out = torch.empty((T, desc.d), dtype=x.dtype, device=x.device)
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(desc), ctypes.byref(wstruct), _ptr(x), T, _ptr(out),
                                           _stream(stream)), "moe_layer_forward_noalloc")
    return out


def moe_workspace_routing(desc: LayerDesc, T: int) -> dict:
    """Byte offsets of the routing moe_layer_forward leaves in its workspace."""
    lay = RoutingLayout()
    _check(lib().moe_workspace_routing(ctypes.byref(desc), T, ctypes.byref(lay)), "moe_workspace_routing")
    return {n: int(getattr(lay, n)) for n, _ in RoutingLayout._fields_}


def routing_views(desc: LayerDesc, T: int, ws: torch.Tensor) -> dict:
    """The routing a completed moe_layer_forward call left in ``ws``, as
    tensor views: ids [T, K] int32, weights [T, K] fp32, counts [E],
    offsets [E + 1], route_src [T*K], route_pos [T*K] (int32)."""
    off = moe_workspace_routing(desc, T)
    K, E, R = desc.K, desc.E, T * desc.K

    def view(name, n, dtype):
        return ws[off[name]: off[name] + 4 * n].view(dtype)

    return {"ids": view("ids", R, torch.int32).view(T, K), "weights": view("weights", R, torch.float32).view(T, K),
            "counts": view("counts", E, torch.int32), "offsets": view("offsets", E + 1, torch.int32),
            "route_src": view("route_src", R, torch.int32), "route_pos": view("route_pos", R, torch.int32)}


def moe_pack_weight(w: torch.Tensor, kind: int, out=None, stream=None, fp4: bool = False) -> torch.Tensor:
    """Pack [R, C] or [G, R, C] plain row-major device matrices into the
    library's weight layout (kind MOE_PACK_OUT_IN or MOE_PACK_NEURON_MAJOR).
    The result keeps the logical shape; only the element order changes.
    fp4: ``w`` holds MXFP4 codes two per byte (its last dimension is C / 2)."""
    w = w.contiguous()
    G, R, C = (1, *w.shape) if w.dim() == 2 else w.shape
    dt = _wdt(w)
    if fp4:
        C, dt = 2 * C, MOE_MXFP4
    if out is None:
        out = torch.empty_like(w)
    _check(lib().moe_pack_weight(_ptr(w), dt, G, R, C, kind, _ptr(out), _stream(stream)),
           "moe_pack_weight")
    return out


# layout each weight is packed in; the router weight and bias stay plain
PACK_KIND = {
    "w_up": MOE_PACK_OUT_IN, "w_down_t": MOE_PACK_NEURON_MAJOR,
    "w_up_shared": MOE_PACK_OUT_IN, "w_down_shared_t": MOE_PACK_NEURON_MAJOR,
    "w_latent_in": MOE_PACK_OUT_IN, "w_latent_out": MOE_PACK_OUT_IN,
}


# the expert matrices FP8 experts hold as codes, and their scale fields
FP8_SCALE_KEY = {"w_up": "w_up_scale", "w_down": "w_down_scale",
                 "w_up_shared": "w_up_shared_scale", "w_down_shared": "w_down_shared_scale"}


# MXFP4 experts: the E8M0 scale field of each expert matrix
MXFP4_SCALE_KEY = {"w_up": "w_up_e8", "w_down": "w_down_e8",
                   "w_up_shared": "w_up_shared_e8", "w_down_shared": "w_down_shared_e8"}


def device_weights(w_cpu: dict, device, expert_dtype: str | None = None) -> dict:
    """Upload a weight dict in PyTorch storage order and pack it for the
    library: the down projections are transposed to neuron-major on the
    host, then every expert, shared and latent matrix is packed on the
    device (done once at load).  expert_dtype "fp8": the routed and shared
    expert matrices are quantised per output channel on the device first
    (moe_quantize_fp8 on the [out, in] storage), the down codes transposed
    to neuron-major, and the scales stored under the w_*_scale keys.
    expert_dtype "mxfp4": each expert matrix is quantised by
    moe_quantize_mxfp4 on its [out, in] storage (scales under the w_*_e8
    keys); the down projections keep their codes twice, packed [OUT_IN]
    under w_down / w_down_shared and transposed to neuron-major under
    w_down_t / w_down_shared_t.  expert_dtype "mxfp4_a8" (W4A8): the same
    weights as "mxfp4"."""
    out = {}
    for k, v in w_cpu.items():
        if expert_dtype in ("mxfp4", "mxfp4_a8") and k in MXFP4_SCALE_KEY:
            codes, out[MXFP4_SCALE_KEY[k]] = moe_quantize_mxfp4(v.contiguous().to(device))
            out[k] = moe_pack_weight(codes, MOE_PACK_OUT_IN, fp4=True)
            if k in ("w_down", "w_down_shared"):
                out[k + "_t"] = moe_pack_weight(fp4_transpose(codes), MOE_PACK_NEURON_MAJOR, fp4=True)
            continue
        if expert_dtype == "fp8" and k in FP8_SCALE_KEY:
            codes, out[FP8_SCALE_KEY[k]] = moe_quantize_fp8(v.contiguous().to(device))
            if k == "w_down":
                k, codes = "w_down_t", codes.transpose(1, 2)
            elif k == "w_down_shared":
                k, codes = "w_down_shared_t", codes.t()
            out[k] = moe_pack_weight(codes.contiguous(), PACK_KIND[k])
            continue
        if k == "w_down":
            k, v = "w_down_t", v.transpose(1, 2)
        elif k == "w_down_shared":
            k, v = "w_down_shared_t", v.t()
        v = v.contiguous().to(device)
        if k in PACK_KIND:
            v = moe_pack_weight(v, PACK_KIND[k])
        out[k] = v
    torch.cuda.current_stream(device).synchronize()
    return out


# ---------------------------------------------------------------------------
# backward pass
# ---------------------------------------------------------------------------

def device_weights_bwd(w_cpu: dict, device) -> dict:
    """The second packing the backward pass reads: the up and down matrices
    (and a latent layer's projections) from their PyTorch storage, packed
    neuron-major (MOE_PACK_NEURON_MAJOR)."""
    out = {}
    for k, nk in (("w_up", "w_up_nm"), ("w_down", "w_down_nm"), ("w_up_shared", "w_up_shared_nm"),
                  ("w_down_shared", "w_down_shared_nm"), ("w_latent_in", "w_latent_in_nm"),
                  ("w_latent_out", "w_latent_out_nm")):
        if w_cpu.get(k) is not None:
            out[nk] = moe_pack_weight(w_cpu[k].contiguous().to(device), MOE_PACK_NEURON_MAJOR)
    torch.cuda.current_stream(device).synchronize()
    return out


def moe_backward_workspace_size(desc: LayerDesc, T: int) -> int:
    return lib().moe_backward_workspace_size(ctypes.byref(desc), T)


def moe_layer_forward_train(desc: LayerDesc, wstruct: LayerWeights, x: torch.Tensor, ws: torch.Tensor, out=None,
                            stream=None) -> torch.Tensor:
    """The layer output, keeping the forward state in ``ws`` (a backward
    workspace) for ``moe_layer_backward(..., saved=True)``."""
    T = x.shape[0]
    if out is None:
        out = torch.empty((T, desc.d), dtype=x.dtype, device=x.device)
    _check(lib().moe_layer_forward_train(ctypes.byref(desc), ctypes.byref(wstruct), _ptr(x), T, _ptr(out), _ptr(ws),
                                         ws.numel(), _stream(stream)), "moe_layer_forward_train")
    return out


def moe_layer_backward(desc: LayerDesc, wstruct: LayerWeights, wbwd: dict, x: torch.Tensor, dy: torch.Tensor,
                       grads=None, ws=None, stream=None, events=None, saved=False) -> dict:
    """Gradients of the layer given dY (see moe_layer_backward in moe.h):
    dx [T, d] bf16 and fp32 dw_router [E, d], dw_up [E, F, d_e], dw_down
    [E, d_e, F] (d_e = d_latent for a latent layer, else d), dw_up_shared
    [F_s, d], dw_down_shared [d, F_s], with the fused front
    (MOE_FLAG_PRENORM_RESIDUAL; x is then the hidden state) dw_norm [d], and
    for a latent layer dw_latent_in [L, d] and dw_latent_out [d, L]."""
    T = x.shape[0]
    dev = x.device
    E, F, Fs, d, L = desc.E, desc.F, desc.F_shared, desc.d, desc.d_latent
    de = L or d
    if grads is None:
        grads = {"dx": torch.empty((T, d), dtype=x.dtype, device=dev),
                 "dw_router": torch.empty((E, d), dtype=torch.float32, device=dev),
                 "dw_up": torch.empty((E, F, de), dtype=torch.float32, device=dev),
                 "dw_down": torch.empty((E, de, F), dtype=torch.float32, device=dev)}
        if Fs:
            grads["dw_up_shared"] = torch.empty((Fs, d), dtype=torch.float32, device=dev)
            grads["dw_down_shared"] = torch.empty((d, Fs), dtype=torch.float32, device=dev)
        if desc.flags & MOE_FLAG_PRENORM_RESIDUAL:
            grads["dw_norm"] = torch.empty((d,), dtype=torch.float32, device=dev)
        if L:
            grads["dw_latent_in"] = torch.empty((L, d), dtype=torch.float32, device=dev)
            grads["dw_latent_out"] = torch.empty((d, L), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(moe_backward_workspace_size(desc, T), dev)
    wb = LayerWeightsBwd(*[(wbwd[n].data_ptr() if wbwd.get(n) is not None else None)
                           for n, _ in LayerWeightsBwd._fields_])
    gs = LayerGrads(*[(grads[n].data_ptr() if grads.get(n) is not None else None) for n, _ in LayerGrads._fields_])
    if events is None:
        fn = lib().moe_layer_backward_saved if saved else lib().moe_layer_backward
        st = fn(ctypes.byref(desc), ctypes.byref(wstruct), ctypes.byref(wb), _ptr(x), _ptr(dy),
                T, ctypes.byref(gs), _ptr(ws), ws.numel(), _stream(stream))
    else:
        st = lib().moe_layer_backward_timed(ctypes.byref(desc), ctypes.byref(wstruct), ctypes.byref(wb), _ptr(x),
                                            _ptr(dy), T, ctypes.byref(gs), _ptr(ws), ws.numel(), _stream(stream),
                                            events, int(bool(saved)))
    _check(st, "moe_layer_backward")
    return grads
