"""Parity at the full sizes of the workloads, in the launch configuration the
benchmark times: the Nano prefill layer (T=4096), the Nano decode batches
(T = 1, 4, 16, 64, decode path), the Super latent layer (T=2048, 512 experts,
top-22) and the Nano load-imbalance stress layer (T=16384, log-Zipf bias,
8 groups of which 4 are kept, 1 % exact-tie rows).

Routing ids are compared on every row (near-ties counted), dispatch offsets
and maps bit-exactly, outputs on sampled rows that the token-major oracle
computes one by one (every row for the decode batches).
"""
import time

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


def log(*a):
    print(*a, flush=True)


_CASES = {}


def _case(cfg):
    """Weights and inputs of a config, generated once per process."""
    key = (cfg.name, cfg.T, cfg.seed, cfg.x_seed)
    if key not in _CASES:
        t0 = time.time()
        _CASES.clear()  # keep one full-size weight set resident at a time
        torch.cuda.empty_cache()
        _CASES[key] = H.make_case(cfg)
        log(f"[full] generated {cfg.name} T={cfg.T} in {time.time() - t0:.1f} s")
    return _CASES[key]


def _check_full(case, flags=0, n_sample=32, cache=True, extra_rows=()):
    cfg = case.cfg
    p = cfg.params()
    t0 = time.time()
    y = H.run_fused(case, flags)
    z = M.moe_router_logits(case.x_dev, case.w_dev["w_router"])
    ids, w = M.moe_route(z, case.w_dev["bias"], cfg.K, cfg.n_group, cfg.topk_group,
                         cfg.norm_topk_prob, cfg.routed_scaling_factor)
    counts, offsets, rs, rp = M.moe_dispatch(ids, cfg.E)
    torch.cuda.synchronize()
    ids_g = _np(ids)
    x64 = synth.to_f64(case.x_cpu)
    w64 = H.oracle_weights(case.w_cpu, lazy=True, cache=cache)
    # routing on every row
    logits = O.router_logits(x64, w64["w_router"])
    ids_ref, w_ref, info = O.route(logits, w64.get("bias"), cfg.n_group, cfg.topk_group, cfg.K,
                                   cfg.norm_topk_prob, cfg.routed_scaling_factor)
    bad, near, near_diff = H.compare_ids(ids_g, ids_ref, info)
    assert len(bad) == 0, ("id mismatch on rows", bad[:10])
    ok = np.all(ids_g == ids_ref, axis=1)
    werr = np.max(np.abs(_np(w)[ok] - w_ref[ok]))
    assert werr <= 1e-5 * cfg.routed_scaling_factor, werr
    # dispatch of the GPU's ids is exact
    c, o, s, pp = O.dispatch(ids_g, cfg.E)
    assert np.array_equal(_np(counts), c) and np.array_equal(_np(offsets), o)
    assert np.array_equal(_np(rs), s) and np.array_equal(_np(rp), pp)
    # outputs on sampled rows
    rng = np.random.default_rng(cfg.T + cfg.E)
    if n_sample >= cfg.T:
        rows = np.arange(cfg.T)
    else:
        rows = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, n_sample, replace=False),
                                         np.asarray(extra_rows, dtype=np.int64)]))
    # near-tie rows are left out of the output check: the fused path's own
    # fp32 router may resolve them the other way
    rows = rows[(info["gap"][rows] >= H.NEAR_TIE) | info["exact_tie"][rows]]
    gw = O.gate_weights(O.sigmoid(logits[rows]), ids_g[rows], cfg.norm_topk_prob,
                        cfg.routed_scaling_factor)
    out_ref = H.oracle_rows_with_ids(p, x64, w64, rows, ids_g[rows], gw)
    yg = _np(y.float())[rows].astype(np.float64)
    rel, glob = H.row_error(yg, out_ref)
    hist = np.bincount(ids_g.reshape(-1), minlength=cfg.E)
    log(f"[full] {cfg.name} T={cfg.T}: max row rel err {rel:.3e} (global {glob:.3e}) on "
        f"{len(rows)} rows; near-tie rows {len(near)} (differing {len(near_diff)}); "
        f"max/mean expert load {hist.max() / max(hist.mean(), 1e-9):.1f}; {time.time() - t0:.1f} s")
    assert rel <= H.TOL[cfg.dtype], rel
    return ids_g, logits


@pytest.mark.timeout(900)
def test_nano_prefill_full_size():
    case = _case(synth.NANO_PREFILL)
    _check_full(case, n_sample=32)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", synth.DECODE_T)
def test_nano_decode_full_size(T):
    base = _case(synth.NANO_PREFILL)
    cfg = synth.NANO_DECODE.with_T(T)
    x = synth.make_inputs(cfg, base.w_cpu)["x"]
    case = H.Case(cfg, base.w_cpu, x, base.w_dev, x.to(DEV))
    _check_full(case, flags=M.MOE_FLAG_ZERO_SKIP_DOWN, n_sample=T)


@pytest.mark.timeout(900)
def test_super_latent_full_size():
    case = _case(synth.SUPER_LATENT)
    _check_full(case, n_sample=12, cache=False)


def _tie_logits(cfg, z32, bias, pairs, rows):
    """Edit rows of fp32 logits so that a twin pair (i < j, equal bias) ties
    exactly at the K-th position: both logits set to the one fp32 value whose
    sigmoid lands between the K-1-th and K-th largest eligible corrected
    scores of the other experts.  Rows where no pair can be placed so (the
    group choice would change, or the pair would not sit at K and K+1) keep
    their logits.  Returns the edited logits and {row: (i, j)}."""
    z = z32.copy()
    placed = {}
    b32 = bias.astype(np.float32)
    K = cfg.K
    for t in rows:
        for i, j in pairs:
            zt = z[t].astype(np.float64)
            s_, s32, c32, _ = O.decision_scores(zt[None], b32)
            elig = O.eligible_experts(c32, cfg.n_group, cfg.topk_group)[0].copy()
            others = np.where(elig, c32[0].astype(np.float64), -np.inf)
            others[[i, j]] = -np.inf
            srt = -np.sort(-others)
            theta = 0.5 * (srt[K - 2] + srt[K - 1])
            q = theta - float(b32[i])
            if not (0.0 < q < 1.0):
                continue
            zi = np.float32(np.log(q / (1.0 - q)))
            trial = z[t].copy()
            trial[i] = trial[j] = zi
            ids, _, info = O.route(trial[None].astype(np.float64), b32, cfg.n_group, cfg.topk_group, K,
                                   cfg.norm_topk_prob, cfg.routed_scaling_factor)
            if info["exact_tie"][0] and ids[0, K - 1] == i and j not in ids[0]:
                z[t] = trial
                placed[int(t)] = (int(i), int(j))
                break
    return z, placed


@pytest.mark.timeout(900)
def test_nano_stress_full_size_and_exact_ties():
    cfg = synth.NANO_STRESS
    case = _case(cfg)
    inp = synth.make_inputs(cfg, case.w_cpu)  # for its twin pairs and tie rows
    ids_g, logits = _check_full(case, n_sample=24, extra_rows=inp["tie_rows"][:8])
    # exact ties at the top-K boundary, exercised through moe_route on the
    # same fp32 logits the oracle sees
    z32 = logits.astype(np.float32)
    bias = case.w_cpu["bias"].numpy()
    z_t, placed = _tie_logits(cfg, z32, bias, inp["twin_pairs"], inp["tie_rows"])
    log(f"[full] stress: exact ties placed on {len(placed)} of {len(inp['tie_rows'])} rows")
    assert len(placed) >= 0.9 * len(inp["tie_rows"]), len(placed)
    ids, w = M.moe_route(torch.tensor(z_t, device=DEV), case.w_dev["bias"], cfg.K, cfg.n_group,
                         cfg.topk_group, cfg.norm_topk_prob, cfg.routed_scaling_factor)
    torch.cuda.synchronize()
    ids = _np(ids)
    ref, _, info = O.route(z_t.astype(np.float64), bias, cfg.n_group, cfg.topk_group, cfg.K,
                           cfg.norm_topk_prob, cfg.routed_scaling_factor)
    for t, (i, j) in placed.items():
        assert ids[t, cfg.K - 1] == i and j not in ids[t], (t, i, j, ids[t])
        assert np.array_equal(ids[t], ref[t]), (t, ids[t], ref[t])
    bad, near, near_diff = H.compare_ids(ids, ref, info)
    assert len(bad) == 0, bad[:10]
