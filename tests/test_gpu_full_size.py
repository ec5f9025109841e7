"""Parity at the full sizes of the workloads, in the launch configuration the
benchmark times: the Nano prefill layer (T=4096), the Nano decode batches
(T = 1, 4, 16, 64, decode path), the Super latent layer (T=2048, 512 experts,
top-22) and the Nano load-imbalance stress layer (T=16384, log-Zipf bias,
8 groups of which 4 are kept, 1 % exact-tie rows).

Every row is compared: the fused call's own routing ids (near-ties
counted), gate weights, dispatch offsets and maps bit-exactly, and outputs
by row L2 error and per-row element error against the oracle's expert-major
forward with float64 experts converted one at a time.
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


def _check_full(case, flags=0):
    """Every row of a full-size call against the oracle's expert-major
    forward (float64 experts converted one at a time, uncached): the fused
    call's own ids, gates and dispatch, and its output by row L2 and per
    element (see ``_harness.check_layer``).  Returns the GPU's ids and the
    oracle's logits."""
    cfg = case.cfg
    y, rt, ref = H.check_layer(case, flags, lazy=True, cache=False)
    hist = np.bincount(rt["ids"].reshape(-1), minlength=cfg.E)
    log(f"[full] {cfg.name} T={cfg.T}: max/mean expert load {hist.max() / max(hist.mean(), 1e-9):.1f}")
    return rt["ids"], ref["logits"]


@pytest.mark.timeout(900)
def test_nano_prefill_full_size():
    case = _case(synth.NANO_PREFILL)
    _check_full(case)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", synth.DECODE_T)
def test_nano_decode_full_size(T):
    base = _case(synth.NANO_PREFILL)
    cfg = synth.NANO_DECODE.with_T(T)
    x = synth.make_inputs(cfg, base.w_cpu)["x"]
    case = H.Case(cfg, base.w_cpu, x, base.w_dev, x.to(DEV))
    _check_full(case, flags=M.MOE_FLAG_ZERO_SKIP_DOWN)


@pytest.mark.timeout(900)
def test_super_latent_full_size():
    case = _case(synth.SUPER_LATENT)
    _check_full(case)


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
    ids_g, logits = _check_full(case)
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
