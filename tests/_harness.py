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


def compare_ids(ids_gpu, ids_ref, info):
    """Rows whose boundary gap is >= NEAR_TIE, or whose boundary is an exact
    tie of identical inputs, must match exactly.  Returns (mismatching
    required rows, near-tie rows, near-tie rows that differ)."""
    ids_gpu = np.asarray(ids_gpu)
    ids_ref = np.asarray(ids_ref)
    required = (info["gap"] >= NEAR_TIE) | info["exact_tie"]
    diff = np.any(ids_gpu != ids_ref, axis=1)
    return (np.nonzero(diff & required)[0], np.nonzero(~required)[0],
            np.nonzero(diff & ~required)[0])


def oracle_rows_with_ids(p, x64, w64, rows, ids, weights):
    """Layer output of the given rows computed by the oracle's expert and
    combine functions with the given ids and weights (used to re-check
    near-tie rows where the GPU chose differently)."""
    latent = bool(p.get("d_latent", 0))
    w64 = O.quantised_expert_weights(w64, p.get("expert_dtype"))
    out = []
    for i, t in enumerate(rows):
        xt = x64[t]
        xe = xt @ w64["w_latent_in"].T if latent else xt
        acc = np.zeros(xe.shape[0])
        for k in np.argsort(ids[i], kind="stable"):
            e = int(ids[i][k])
            acc += weights[i][k] * O.expert_mlp(xe[None, :], w64["w_up"][e], w64["w_down"][e])[0]
        if latent:
            acc = acc @ w64["w_latent_out"].T
        if p.get("F_shared", 0):
            acc += O.shared_expert(xt[None, :], w64["w_up_shared"], w64["w_down_shared"])[0]
        out.append(acc)
    return np.array(out)
