"""Test harness: builds seeded inputs, runs the HIP path through the C ABI
binding and the CPU oracle side by side, and compares them.

Test infrastructure only (it imports the oracle).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import oracle.moe_oracle as O
import routed_relu_expert_amd as M
from routed_relu_expert_amd import synth

NEAR_TIE = 1e-5          # boundary gap below which a row's ids are not required to match
TOL = {"bf16": 2e-2, "f32": 1e-4}


class LazyExperts:
    """Per-expert float64 view of a [E, ...] CPU tensor, converted on demand
    (the full-size weights would not fit in float64 at once)."""

    def __init__(self, t: torch.Tensor, cache: bool = True):
        self.t = t
        self.cache = cache
        self._cache = {}

    def __len__(self):
        return self.t.shape[0]

    def __getitem__(self, e):
        e = int(e)
        if not self.cache:
            return self.t[e].to(torch.float64).numpy()
        if e not in self._cache:
            self._cache[e] = self.t[e].to(torch.float64).numpy()
        return self._cache[e]


def oracle_weights(w_cpu: dict, lazy: bool = False, cache: bool = True) -> dict:
    out = {}
    for k, v in w_cpu.items():
        if k in ("w_up", "w_down") and lazy:
            out[k] = LazyExperts(v, cache)
        else:
            out[k] = v.to(torch.float64).numpy()
    return out


def small_config(**kw) -> synth.LayerConfig:
    base = dict(name="small", T=300, d=512, E=16, K=4, n_group=1, topk_group=1, F=384,
                F_shared=256, routed_scaling_factor=2.5, dtype="bf16", seed=11, x_seed=12,
                std_router=512 ** -0.5, std_up=512 ** -0.5, std_down=384 ** -0.5,
                std_up_shared=512 ** -0.5, std_down_shared=256 ** -0.5)
    base.update(kw)
    return synth.LayerConfig(**base)


@dataclasses.dataclass
class Case:
    cfg: synth.LayerConfig
    w_cpu: dict
    x_cpu: torch.Tensor
    w_dev: dict
    x_dev: torch.Tensor


def make_case(cfg: synth.LayerConfig, device="cuda", bias=None) -> Case:
    w = synth.make_weights(cfg)
    inp = synth.make_inputs(cfg, w)
    if "bias" in inp:
        w["bias"] = inp["bias"]
    if bias is not None:
        w["bias"] = bias
    wd = M.device_weights(w, device, expert_dtype=cfg.expert_dtype or None)
    return Case(cfg, w, inp["x"], wd, inp["x"].to(device))


def act_code(cfg):
    return M.MOE_BF16 if cfg.dtype == "bf16" else M.MOE_F32


def run_fused(case: Case, flags=0, out=None):
    desc = M.make_desc(case.cfg.params(), act_code(case.cfg), flags)
    ws = M.make_weights_struct(case.w_dev)
    y = M.moe_layer_forward(desc, ws, case.x_dev, out=out)
    torch.cuda.synchronize()
    return y


def row_error(y, y_ref):
    return O.row_relative_error(y, y_ref)


def compare_ids(ids_gpu, ids_ref, info, band=NEAR_TIE):
    """Rows whose boundary gap is >= band (NEAR_TIE, or a per-row array), or
    whose boundary is an exact tie of identical inputs, must match exactly.
    Returns (mismatching required rows, near-tie rows, near-tie rows that
    differ)."""
    ids_gpu = np.asarray(ids_gpu)
    ids_ref = np.asarray(ids_ref)
    required = (info["gap"] >= band) | info["exact_tie"]
    diff = np.any(ids_gpu != ids_ref, axis=1)
    return (np.nonzero(diff & required)[0], np.nonzero(~required)[0],
            np.nonzero(diff & ~required)[0])


def oracle_rows_with_ids(p, x64, w64, rows, ids, weights):
    """Layer output of the given rows computed by the oracle's expert and
    combine functions with the given ids and weights (used to re-check
    near-tie rows where the GPU chose differently)."""
    latent = bool(p.get("d_latent", 0))
    w64 = O.quantised_expert_weights(w64, p.get("expert_dtype"))
    aq = O.activation_quantiser(p.get("expert_dtype"), p.get("act_dtype", "bf16"))
    out = []
    for i, t in enumerate(rows):
        xt = x64[t]
        xe = xt @ w64["w_latent_in"].T if latent else xt
        acc = np.zeros(xe.shape[0])
        for k in np.argsort(ids[i], kind="stable"):
            e = int(ids[i][k])
            acc += weights[i][k] * O.expert_mlp(xe[None, :], w64["w_up"][e], w64["w_down"][e], aq)[0]
        if latent:
            acc = acc @ w64["w_latent_out"].T
        if p.get("F_shared", 0):
            acc += O.shared_expert(xt[None, :], w64["w_up_shared"], w64["w_down_shared"], aq)[0]
        out.append(acc)
    return np.array(out)


# ---------------------------------------------------------------------------
# RMSNorm in front of the layer: how far the GPU's fp32 evaluation can be
# from the oracle's float64 definition
# ---------------------------------------------------------------------------

U32 = 2.0 ** -24


def rmsnorm_rel_bound(d):
    """Relative error bound of the GPU RMSNorm's fp32 value before its one
    rounding to the activation dtype.  The kernel adds n = 8 * ceil(d / 512)
    squares per lane in sequence, folds the 64 lane sums in 6 levels,
    divides by d, adds eps (all terms non-negative), takes a correctly
    rounded square root and reciprocal and two products: to first order
    (n + 8) / 2 + 4 units of 2^-24; one more unit covers the second-order
    terms."""
    n = 8 * -(-d // 512)
    return ((n + 8) / 2 + 5) * U32


def bf16_spacing(v):
    """Spacing of bfloat16 values at |v| (its binade's ulp)."""
    _, e = np.frexp(np.asarray(v, dtype=np.float64))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def rmsnorm_may_round_differently(v_exact, d, act):
    """Elements whose exact norm value lies within the GPU's error bound of
    a rounding midpoint of the activation dtype: only these may round to a
    neighbouring value on the GPU (every element, for fp32 outputs)."""
    v = np.asarray(v_exact, dtype=np.float64)
    if act == "f32":
        return np.ones(v.shape, dtype=bool)
    q = bf16_spacing(v)
    r = np.abs(v) / q
    dist = np.abs(r - np.floor(r) - 0.5) * q
    return dist <= rmsnorm_rel_bound(d) * np.abs(v)


def prenorm_band(v_exact, w_router, act):
    """Per-row near-tie band of the router boundary when the layer input is
    the GPU's own RMSNorm: 1e-5 plus the most the logits can move through
    input elements that may round differently (one bfloat16 step each; for
    fp32 outputs the relative error bound on every element).  A logit moved
    by delta moves a sigmoid by at most delta / 4, the K-th minus (K+1)-th
    score gap by delta / 2 and a top-two group score gap by delta."""
    v = np.asarray(v_exact, dtype=np.float64)
    d = v.shape[1]
    if act == "f32":
        step = (rmsnorm_rel_bound(d) + 2 * U32) * np.abs(v)
    else:
        step = np.where(rmsnorm_may_round_differently(v, d, act), bf16_spacing(v), 0.0)
    delta = (step @ np.abs(np.asarray(w_router, dtype=np.float64)).T).max(axis=1)
    return NEAR_TIE + delta


def elementwise_row_error(y, y_ref):
    """Per row, max_j |y_tj - yref_tj| / max_j |yref_tj| (absolute for an
    all-zero reference row): a single wrong element of a row shows here
    even where the row's L2 error hides it."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y.size == 0:
        return np.zeros(y.shape[0])
    num = np.max(np.abs(y - y_ref), axis=1)
    den = np.max(np.abs(y_ref), axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def run_fused_routing(case: Case, flags=0, out=None):
    """The fused layer's output and the routing it computed, read from its
    workspace (moe_workspace_routing): ids, weights, counts, offsets,
    route_src, route_pos as numpy arrays."""
    desc = M.make_desc(case.cfg.params(), act_code(case.cfg), flags)
    T = case.x_dev.shape[0]
    ws = torch.empty(max(M.moe_workspace_size(desc, T), 1), dtype=torch.uint8, device=case.x_dev.device)
    y = M.moe_layer_forward(desc, M.make_weights_struct(case.w_dev), case.x_dev, out=out, ws=ws)
    torch.cuda.synchronize()
    views = M.routing_views(desc, T, ws)
    return y, {k: v.cpu().numpy() for k, v in views.items()}


def check_layer(case: Case, flags=0, lazy=False, cache=True, extra_log=""):
    """The fused layer against the oracle on every row.

    * ids of the fused call itself (read from its workspace) bit-exact on
      every row outside the near-tie band; its gate weights within 1e-5 rsf
      on those rows;
    * its counts, offsets and route maps: the oracle's dispatch of those ids
      (bit-exact), and the oracle's own when no near tie went the other way;
    * outputs: max row-relative L2 error and max per-row element error
      (``elementwise_row_error``) both within the dtype's tolerance, rows
      whose near tie went the other way recomputed by the oracle with the
      GPU's choice.
    Returns (y, routing, oracle result)."""
    import time
    cfg = case.cfg
    p = cfg.params()
    t0 = time.time()
    x64 = synth.to_f64(case.x_cpu)
    w64 = oracle_weights(case.w_cpu, lazy=lazy, cache=cache)
    y, rt = run_fused_routing(case, flags)
    ref = O.layer_forward(p, x64, w64)
    prenorm = bool(p.get("prenorm_residual"))
    xl64 = x64
    band = NEAR_TIE
    if prenorm:
        act = p["act_dtype"]
        v = O.rms_norm_exact(x64, w64["w_norm"], p["norm_eps"])
        xl64 = O.round_once(v, act)
        band = prenorm_band(v, w64["w_router"], act)
    info = ref["route_info"]
    ids_g = rt["ids"]
    bad, near, near_diff = compare_ids(ids_g, ref["ids"], info, band)
    assert len(bad) == 0, ("id mismatch on rows", bad[:10], ids_g[bad[:3]], ref["ids"][bad[:3]])
    rsf = cfg.routed_scaling_factor
    same = np.all(ids_g == ref["ids"], axis=1) & ((info["gap"] >= band) | info["exact_tie"])
    if same.any():
        # 1e-5 rsf (the fused path's own fp32 logits); with the fused norm in
        # front, plus what a logit move of delta can do to a gate: each
        # sigmoid moves by delta / 4, so a normalised gate rsf s_k / S by at
        # most rsf (delta / 4) (1 + K) / S, an unnormalised one by rsf delta / 4
        delta = np.asarray(band, dtype=np.float64) - NEAR_TIE
        if cfg.norm_topk_prob:
            s_sel = np.take_along_axis(O.sigmoid(ref["logits"]), ref["ids"].astype(np.int64), axis=1).sum(axis=1)
            wtol = rsf * (1e-5 + delta / 4 * (1 + cfg.K) / s_sel)
        else:
            wtol = rsf * (1e-5 + delta / 4) * np.ones(cfg.T)
        werr = np.max(np.abs(rt["weights"] - ref["weights"]), axis=1)
        assert np.all(werr[same] <= wtol[same]), float(np.max(werr[same] - wtol[same]))
    # dispatch of the GPU's own ids: exact
    cf = p.get("capacity_factor", 0)
    if not cf:
        c, o, s_, pp = O.dispatch(ids_g, cfg.E)
        assert np.array_equal(rt["counts"], c) and np.array_equal(rt["offsets"], o)
        assert np.array_equal(rt["route_src"], s_) and np.array_equal(rt["route_pos"], pp)
    if len(near_diff) == 0:
        assert np.array_equal(rt["offsets"], ref["offsets"])
        assert np.array_equal(rt["route_pos"], ref["route_pos"])
        n_acc = int(ref["offsets"][-1])
        assert np.array_equal(rt["route_src"][:n_acc], ref["route_src"][:n_acc])
    out_ref = ref["out"]
    if len(near_diff):
        assert not cf, "a capacity case must not have near ties that flip"
        rows = near_diff
        s64 = O.sigmoid(O.router_logits(xl64[rows], w64["w_router"]))
        gi = ids_g[rows]
        gw = O.gate_weights(s64, gi, cfg.norm_topk_prob, rsf)
        out_ref = out_ref.copy()
        out_ref[rows] = oracle_rows_with_ids(p, xl64, w64, rows, gi, gw)
        if prenorm:
            out_ref[rows] += x64[rows]
    yg = y.float().cpu().numpy().astype(np.float64)
    rel, glob = row_error(yg, out_ref)
    elem = elementwise_row_error(yg, out_ref)
    emax = float(elem.max()) if elem.size else 0.0
    tol = TOL[cfg.dtype]
    print(f"{cfg.name} T={cfg.T}: rows compared = {cfg.T}; max row rel err {rel:.3e}, max row element "
          f"err {emax:.3e} (global {glob:.3e}); near-tie rows {len(near)} (differing {len(near_diff)}); "
          f"{time.time() - t0:.1f} s {extra_log}", flush=True)
    assert rel <= tol, rel
    assert emax <= tol, (emax, int(np.argmax(elem)))
    return y, rt, ref
