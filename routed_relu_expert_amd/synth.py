"""Seeded synthetic inputs for the routed ReLU^2 MoE layer.

This module holds no arithmetic of the method: it only draws random
weights and activations with fixed seeds, shapes and distributions, and
casts them to the activation dtype.  Both the HIP path and the CPU oracle
receive exactly these values.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` stream per config):

* weight draw order, in PyTorch storage shapes, on the stream
  ``PCG64(seed)``: router ``W_r [E, d]``, bias ``b [E]``,
  ``W_up [E, F, d_e]``, ``W_down [E, d_e, F]``, shared ``W_up_s [F_s, d]``,
  ``W_down_s [d, F_s]``, then for a latent layer ``W_lin [L, d]``,
  ``W_lout [d, L]``;
* activations on their own stream ``PCG64(SeedSequence([x_seed, 1]))``:
  ``x [T, d]``, then any further decode batches, then the stress config's
  twin pairs and tie rows;
* normal draws are ``standard_normal(dtype=float32) * float32(std)``;
  uniform draws ``uniform(lo, hi).astype(float32)``;
* bf16 tensors are cast from float32 by round-to-nearest-even
  (``torch.Tensor.to(torch.bfloat16)`` on the CPU); the router weight and
  bias stay float32.

Shapes follow the Nemotron Nano layer (128 routed experts plus one shared,
6 per token, widths 2688 / 1856 / 3712) and the Super latent layer (512
experts, top-22, latent 1024, expert up 2688x1024 / down 1024x2688, shared
5376 on 4096).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    d: int
    E: int
    K: int
    n_group: int
    topk_group: int
    F: int
    F_shared: int
    routed_scaling_factor: float
    dtype: str                 # "f32" or "bf16": activations and expert weights
    seed: int                  # weight stream
    x_seed: int                # activation stream key
    d_latent: int = 0
    norm_topk_prob: int = 1
    std_router: float = 0.02
    std_up: float = 0.02
    std_down: float = 0.02
    std_up_shared: float = 0.02
    std_down_shared: float = 0.02
    std_latent_in: float = 0.0
    std_latent_out: float = 0.0
    bias_kind: str = "normal"  # "normal" (std 0.01) or "uniform" (+-0.1)
    zipf_tau: float = 0.0      # log-Zipf offsets added to the bias
    n_twin_pairs: int = 0      # experts whose bias is made equal (stress ties)
    tie_row_frac: float = 0.0
    prenorm: bool = False      # RMSNorm in front, residual behind (w_norm drawn last)
    norm_eps: float = 1e-5
    capacity_factor: float = 0.0  # > 0: the capacity-bounded variant
    expert_dtype: str = ""     # "fp8": per-output-channel E4M3; "mxfp4": E2M1 with E8M0 block scales;
                               # "mxfp4_a8": those weights, MXFP8 inputs of both expert products

    @property
    def d_e(self) -> int:
        return self.d_latent or self.d

    @property
    def R(self) -> int:
        return self.T * self.K

    def params(self) -> dict:
        p = {"d": self.d, "E": self.E, "K": self.K, "F": self.F,
             "F_shared": self.F_shared, "d_latent": self.d_latent,
             "n_group": self.n_group, "topk_group": self.topk_group,
             "norm_topk_prob": self.norm_topk_prob,
             "routed_scaling_factor": self.routed_scaling_factor}
        if self.prenorm:
            p.update(prenorm_residual=1, norm_eps=self.norm_eps, act_dtype=self.dtype)
        if self.capacity_factor:
            p["capacity_factor"] = self.capacity_factor
        if self.expert_dtype:
            p["expert_dtype"] = self.expert_dtype
        return p

    def with_T(self, T: int) -> "LayerConfig":
        return dataclasses.replace(self, T=T)


def _fan(n: int) -> float:
    return 1.0 / math.sqrt(n)


TINY_F32 = LayerConfig(
    name="tiny_f32", T=64, d=256, E=8, K=2, n_group=1, topk_group=1, F=512,
    F_shared=512, routed_scaling_factor=1.0, dtype="f32", seed=0, x_seed=0,
    bias_kind="uniform")

NANO_PREFILL = LayerConfig(
    name="nano_prefill", T=4096, d=2688, E=128, K=6, n_group=1, topk_group=1,
    F=1856, F_shared=3712, routed_scaling_factor=2.5, dtype="bf16", seed=1,
    x_seed=1, std_router=_fan(2688), std_up=_fan(2688), std_down=_fan(1856),
    std_up_shared=_fan(2688), std_down_shared=_fan(3712))

# Decode batches reuse the prefill weights (seed 1); x comes from seed 2.
NANO_DECODE = dataclasses.replace(NANO_PREFILL, name="nano_decode", T=64, x_seed=2)
DECODE_T = (1, 4, 16, 64)

SUPER_LATENT = LayerConfig(
    name="super_latent", T=2048, d=4096, E=512, K=22, n_group=1, topk_group=1,
    F=2688, F_shared=5376, routed_scaling_factor=1.0, dtype="bf16", seed=3,
    x_seed=3, d_latent=1024, std_router=_fan(4096), std_up=_fan(1024),
    std_down=_fan(2688), std_up_shared=_fan(4096), std_down_shared=_fan(5376),
    std_latent_in=_fan(4096), std_latent_out=_fan(1024))

# Load-imbalance stress: the prefill weights, x from seed 4, log-Zipf(1.2)
# offsets on the bias, 8 groups of 16 with 4 kept, 1 % exact-tie rows.
NANO_STRESS = dataclasses.replace(
    NANO_PREFILL, name="nano_stress", T=16384, n_group=8, topk_group=4,
    x_seed=4, zipf_tau=1.0, n_twin_pairs=8, tie_row_frac=0.01)

CONFIGS = {c.name: c for c in (TINY_F32, NANO_PREFILL, NANO_DECODE, SUPER_LATENT, NANO_STRESS)}


def _normal(rng, shape, std):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def _act(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.clone()


def zipf_log_offsets(E: int, s: float = 1.2) -> np.ndarray:
    """``log p(e+1)`` for ``p(r) = r^-s / H`` over ranks 1..E (identity rank
    map: expert e has rank e+1)."""
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    p /= p.sum()
    return np.log(p)


def make_weights(cfg: LayerConfig) -> dict:
    """Weights of one config as CPU tensors (router and bias float32, the
    rest in the activation dtype), in PyTorch storage order."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    E, d, F, de, Fs = cfg.E, cfg.d, cfg.F, cfg.d_e, cfg.F_shared
    w = {}
    w["w_router"] = torch.from_numpy(_normal(rng, (E, d), cfg.std_router))
    if cfg.bias_kind == "uniform":
        b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    else:
        b = _normal(rng, (E,), 0.01)
    w["bias"] = torch.from_numpy(b)
    w["w_up"] = _act(_normal(rng, (E, F, de), cfg.std_up), cfg.dtype)
    w["w_down"] = _act(_normal(rng, (E, de, F), cfg.std_down), cfg.dtype)
    if Fs:
        w["w_up_shared"] = _act(_normal(rng, (Fs, d), cfg.std_up_shared), cfg.dtype)
        w["w_down_shared"] = _act(_normal(rng, (d, Fs), cfg.std_down_shared), cfg.dtype)
    if cfg.d_latent:
        L = cfg.d_latent
        w["w_latent_in"] = _act(_normal(rng, (L, d), cfg.std_latent_in), cfg.dtype)
        w["w_latent_out"] = _act(_normal(rng, (d, L), cfg.std_latent_out), cfg.dtype)
    if cfg.prenorm:
        w["w_norm"] = make_norm_weight(cfg)
    return w


def make_norm_weight(cfg: LayerConfig) -> torch.Tensor:
    """The RMSNorm weight [d]: 1 + N(0, 0.1), from a stream of its own
    (key (seed, 3)) so that the other weights do not depend on it."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 3])))
    return _act(np.float32(1.0) + _normal(rng, (cfg.d,), 0.1), cfg.dtype)


def make_inputs(cfg: LayerConfig, weights: dict | None = None, n_batches: int = 1) -> dict:
    """Activations (and the stress-config edits) for ``cfg``.

    Returns ``x`` [T, d] in the activation dtype; for decode configs
    ``x_batches`` holds ``n_batches`` further [T, d] draws of the same
    stream; for the stress config ``bias`` (log-Zipf offsets, twin pairs
    equalised), ``twin_pairs`` [P, 2] and ``tie_rows`` (row indices drawn
    without replacement).
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.x_seed, 1])))
    out = {}
    T = cfg.T
    x = rng.standard_normal((T, cfg.d), dtype=np.float32)
    out["x"] = _act(x, cfg.dtype)
    if n_batches > 1:
        out["x_batches"] = [out["x"]] + [
            _act(rng.standard_normal((T, cfg.d), dtype=np.float32), cfg.dtype)
            for _ in range(n_batches - 1)]
    if cfg.zipf_tau:
        assert weights is not None, "the stress bias is built on the base bias"
        b = weights["bias"].numpy().astype(np.float64)
        b4 = (b + cfg.zipf_tau * zipf_log_offsets(cfg.E)).astype(np.float32)
        # twin pairs inside the groups that usually survive (the first
        # topk_group groups of E / n_group experts)
        span = cfg.topk_group * (cfg.E // cfg.n_group)
        perm = rng.permutation(span)[: 2 * cfg.n_twin_pairs].reshape(-1, 2)
        pairs = np.sort(perm, axis=1).astype(np.int64)
        for i, j in pairs:
            b4[j] = b4[i]
        out["bias"] = torch.from_numpy(b4)
        out["twin_pairs"] = pairs
        n_tie = int(round(cfg.tie_row_frac * T))
        out["tie_rows"] = np.sort(rng.choice(T, size=n_tie, replace=False))
    return out


def to_f64(t) -> np.ndarray:
    """Exact float64 copy of a CPU or GPU tensor (bf16 and fp32 widen
    exactly)."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu", torch.float64).numpy()
