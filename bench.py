#!/usr/bin/env python3
"""Benchmark of the routed ReLU^2 MoE layer forward on one MI355X.

One step = one fused moe_layer_forward (router GEMM, route, dispatch, routed
+ shared up projections with ReLU^2, down projections, combine) over the
Nemotron-Nano-shaped prefill batch: T=4096 tokens, d=2688, 128 experts,
top-6, F=1856, shared F=3712, bf16 activations and expert weights, fp32
router; seeded synthetic inputs resident in HBM before the timed region.

Prints one JSON line: tokens/s of the whole layer, the dominant kernel's
roofline (its time measured with HIP events recorded around it inside the
timed steps), the layer's MFMA and HBM fractions, per-stage times, decode
batches (T = 1, 4, 16, 64) with zero-skipping, the variants (RMSNorm front
and residual, fixed capacity, FP8 expert weights), the backward pass and
the CPU oracle baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
ITEM_ROWS = 16  # rows of one work item of the decode path
GEMM_SOURCE = os.path.join(ROOT, "routed_relu_expert_amd", "csrc", "gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic_nano_prefill.md")


def source_sha256(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(stage):
    """HBM bytes per launch of the grouped GEMM of `stage` ("up"/"down") from
    the rocprofv3 FETCH_SIZE / WRITE_SIZE record under profiles/, or None when
    there is none or it was taken on a different GEMM source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            line = line.strip().lstrip("-* ").replace("`", "")
            if ":" in line:
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("gemm.hip sha256") != source_sha256(GEMM_SOURCE):
        return None
    v = rec.get(f"{stage} traffic bytes per launch")
    return float(v) if v else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles created through the HIP runtime torch already loaded."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            self.ev.append(h)
        self.array = (ctypes.c_void_p * n)(*[e.value for e in self.ev])

    def elapsed_ms(self, i, j):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[i], self.ev[j]) == 0
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def warm_up(step, args, torch):
    """``args.warmup`` untimed steps, then more untimed steps until
    ``args.settle_s`` seconds have passed since the first: under this load
    the GPU's clock ramps up over the first few dozen layer calls, and steps
    timed during the ramp measure the ramp, not the kernels.  Returns the
    number of warm-up steps and their seconds."""
    t0 = time.perf_counter()
    n = 0
    while n < args.warmup or time.perf_counter() - t0 < args.settle_s:
        step()
        n += 1
        if n % 8 == 0 or n >= args.warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return {"steps": n, "seconds": round(time.perf_counter() - t0, 3)}


def routing_counts(M, x, wd, cfg):
    z = M.moe_router_logits(x, wd["w_router"])
    ids, w = M.moe_route(z, wd["bias"], cfg.K, cfg.n_group, cfg.topk_group, cfg.norm_topk_prob,
                         cfg.routed_scaling_factor)
    counts, offsets, rs, rp = M.moe_dispatch(ids, cfg.E)
    return counts, offsets, rs


def routing_report(counts, T):
    """The realised per-expert histogram of a batch (max / mean, CV^2,
    normalised entropy of the route shares) and the rows the grouped GEMMs
    compute beyond an expert's routes: padding to whole 32-row MFMA blocks
    (the kernels skip blocks past an expert's rows) and, for scale, to
    whole 256-row tiles; the shared expert's T rows are included."""
    import math
    R = sum(counts)
    E = len(counts)
    mean = R / E
    var = sum((c - mean) ** 2 for c in counts) / E
    shares = [c / R for c in counts if c > 0]
    ent = abs(sum(p * math.log(p) for p in shares)) / math.log(E) if E > 1 else 1.0
    groups = list(counts) + [T]
    pad32 = sum((-c) % 32 for c in groups if c > 0)
    pad256 = sum((-c) % 256 for c in groups if c > 0)
    rows = R + T
    return {"max_over_mean": max(counts) / mean, "cv2": var / mean ** 2, "normalised_entropy": ent,
            "slack_rows_32": pad32, "slack_rows_32_frac": pad32 / rows,
            "slack_rows_256": pad256, "slack_rows_256_frac": pad256 / rows}


def prefill(args, M, synth, torch):
    cfg = synth.NANO_PREFILL
    log(f"[bench] generating {cfg.name} weights and inputs (seeded)")
    w = synth.make_weights(cfg)
    x_cpu = synth.make_inputs(cfg, w)["x"]
    wd = M.device_weights(w, "cuda")
    x = x_cpu.cuda()
    desc = M.make_desc(cfg.params(), M.MOE_BF16)
    wst = M.make_weights_struct(wd)
    ws = torch.empty(M.moe_workspace_size(desc, cfg.T), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda")
    settled = warm_up(lambda: M.moe_layer_forward(desc, wst, x, out=out, ws=ws), args, torch)

    # timed region: exactly `steps` fused steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        M.moe_layer_forward(desc, wst, x, out=out, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    log(f"[bench] {cfg.name}: {ms:.4f} ms/step (wall {wall / args.steps * 1e3:.4f} ms/step)")

    # per-stage times: events recorded around each stage's kernels inside
    # the same fused call, on the stream the kernels run on
    nst = len(M.STAGES)
    ev = HipEvents(2 * nst)
    stage_ms = [0.0] * nst
    for _ in range(args.steps):
        M.moe_layer_forward(desc, wst, x, out=out, ws=ws, events=ev.array)
        torch.cuda.synchronize()
        for s in range(nst):
            stage_ms[s] += ev.elapsed_ms(2 * s, 2 * s + 1)
    ev.close()
    stage_ms = [v / args.steps for v in stage_ms]

    counts, _, _ = routing_counts(M, x, wd, cfg)
    touched = int((counts > 0).sum().item())
    R = cfg.T * cfg.K
    de = cfg.d_e
    exp_bytes = cfg.F * de * 2  # one projection of one expert, bf16
    flops_up = 2.0 * R * de * cfg.F + 2.0 * cfg.T * cfg.d * cfg.F_shared
    flops_down = 2.0 * R * cfg.F * de + 2.0 * cfg.T * cfg.F_shared * cfg.d
    bytes_up = touched * exp_bytes + cfg.F_shared * cfg.d * 2 + cfg.T * cfg.d * 2
    bytes_down = touched * exp_bytes + cfg.F_shared * cfg.d * 2
    layer_flops = flops_up + flops_down + 2.0 * cfg.T * cfg.d * cfg.E
    layer_bytes = (2 * touched * exp_bytes + 2 * cfg.F_shared * cfg.d * 2 + cfg.E * cfg.d * 4
                   + 2 * cfg.T * cfg.d * 2)
    st = dict(zip(M.STAGES, stage_ms))
    dom = "up" if st["up"] >= st["down"] else "down"
    dom_ms = st[dom]
    dom_bytes = bytes_up if dom == "up" else bytes_down
    dom_flops = flops_up if dom == "up" else flops_down
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    res = {
        "ms_per_step": ms,
        "warmup_settle": settled,
        "tokens_per_s": cfg.T / (ms * 1e-3),
        "stages_ms": {k: round(v, 5) for k, v in st.items()},
        "roofline": {"bound": "hbm", "kernel": f"grouped_gemm_{dom} (gemm_bf16_kernel)",
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(dom),
                     "algorithmic_bytes_per_launch": dom_bytes,
                     "mfma_tflops": dom_flops / (dom_ms * 1e-3) / 1e12,
                     "mfma_frac": dom_flops / (dom_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "layer": {"gflop": layer_flops / 1e9, "algorithmic_gb": layer_bytes / 1e9,
                  "tflops": layer_flops / (ms * 1e-3) / 1e12,
                  "mfma_frac": layer_flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                  "hbm_gbps": layer_bytes / (ms * 1e-3) / 1e9,
                  "hbm_frac": layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                  "roofline_frac": max(layer_flops / (BF16_PEAK_TFLOPS * 1e12),
                                       layer_bytes / (HBM_PEAK_GBPS * 1e9)) / (ms * 1e-3),
                  "experts_touched": touched,
                  "routing": routing_report(counts.cpu().tolist(), cfg.T)},
    }
    return res, cfg, w, x_cpu, wd


def decode(args, M, synth, torch, w_cpu, wd, fmt=None):
    """Decode batches with zero-skipping; weight copies at distinct
    addresses are cycled (8, or 16 for the 4-bit weights) so each step's
    weights come from HBM, not from the 256 MB last-level cache.  fmt
    "fp8": the experts' weights are E4M3 codes with per-output-channel
    scales; "mxfp4": E2M1 codes with an E8M0 scale per 32 inputs (wd from
    device_weights(..., fmt))."""
    cfg0 = synth.NANO_DECODE
    fp8, fp4 = fmt == "fp8", fmt == "mxfp4"
    if fmt:
        cfg0 = synth.dataclasses.replace(cfg0, expert_dtype=fmt)
    wb = 0.5 if fp4 else 1 if fp8 else 2  # bytes per expert weight
    ncopy = 16 if fp4 else 8
    copies = [wd] + [{k: v.clone() for k, v in wd.items()} for _ in range(ncopy - 1)]
    inp = synth.make_inputs(cfg0, w_cpu, n_batches=ncopy)
    xs_all = [t.cuda() for t in inp["x_batches"]]
    out = {}
    for T in args.decode_T:
        cfg = cfg0.with_T(T)
        desc = M.make_desc(cfg.params(), M.MOE_BF16, M.MOE_FLAG_ZERO_SKIP_DOWN)
        wss = [M.make_weights_struct(c) for c in copies]
        xs = [xb[:T].contiguous() for xb in xs_all]
        ws = torch.empty(M.moe_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
        y = torch.empty((T, cfg.d), dtype=torch.bfloat16, device="cuda")
        for i in range(2 * ncopy):
            M.moe_layer_forward(desc, wss[i % ncopy], xs[i % ncopy], out=y, ws=ws)
        torch.cuda.synchronize()
        steps = args.decode_steps
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if args.decode_marks:
            # a spin kernel before and after the eager steps, so that a
            # per-dispatch counter trace can be cut into this batch's steps
            torch.cuda._sleep(1000)
        e0.record()
        for i in range(steps):
            M.moe_layer_forward(desc, wss[i % ncopy], xs[i % ncopy], out=y, ws=ws)
        e1.record()
        if args.decode_marks:
            torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        us_eager = e0.elapsed_time(e1) / steps * 1e3
        # the same steps replayed from HIP graphs (one per weight copy), as a
        # decode loop runs them: no host launch cost between kernels.  Each
        # graph's output is checked bitwise against an eager call.
        graph_ok = None
        us = us_eager
        if not args.decode_marks:
            ys = [torch.empty_like(y) for _ in range(ncopy)]
            graphs = []
            for i in range(ncopy):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    M.moe_layer_forward(desc, wss[i], xs[i], out=ys[i], ws=ws)
                graphs.append(g)
            graph_ok = True
            for i in range(ncopy):
                graphs[i].replay()
                torch.cuda.synchronize()
                ref = M.moe_layer_forward(desc, wss[i], xs[i], ws=ws)
                torch.cuda.synchronize()
                graph_ok &= bool(torch.equal(ref, ys[i]))
            for i in range(2 * ncopy):
                graphs[i % ncopy].replay()
            torch.cuda.synchronize()
            e0.record()
            for i in range(steps):
                graphs[i % ncopy].replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / steps * 1e3
            del graphs
        # weight bytes the step reads: the router (fp32), the up rows of every
        # touched expert and of the shared expert, and the down rows of the
        # neurons that are non-zero for some row of each 16-row work item
        # (items of one expert that has more than 16 rows each read their own
        # live rows); averaged over the batches cycled above
        need = dense = zeros = elems = skipped = rows = 0.0
        for i in range(ncopy):
            x = xs[i]
            counts, offsets, rs = routing_counts(M, x, wd, cfg)
            zc = torch.zeros(2, dtype=torch.int64, device="cuda")
            zs = torch.zeros(2, dtype=torch.int64, device="cuda")
            one = torch.tensor([0, T], dtype=torch.int32, device="cuda")
            f = M.MOE_FLAG_ZERO_SKIP_DOWN
            if fp4:
                M.moe_experts_mxfp4(x, cfg.K, rs, offsets, wd["w_up"], wd["w_up_e8"], wd["w_down_t"], wd["w_down"],
                                    wd["w_down_e8"], flags=f, zero_count=zc)
                M.moe_experts_mxfp4(x, 1, None, one, wd["w_up_shared"][None], wd["w_up_shared_e8"][None],
                                    wd["w_down_shared_t"][None], wd["w_down_shared"][None],
                                    wd["w_down_shared_e8"][None], flags=f, zero_count=zs)
            elif fp8:
                M.moe_experts_fp8(x, cfg.K, rs, offsets, wd["w_up"], wd["w_up_scale"], wd["w_down_t"],
                                  wd["w_down_scale"], flags=f, zero_count=zc)
                M.moe_experts_fp8(x, 1, None, one, wd["w_up_shared"][None], wd["w_up_shared_scale"][None],
                                  wd["w_down_shared_t"][None], wd["w_down_shared_scale"][None], flags=f,
                                  zero_count=zs)
            else:
                M.moe_experts(x, cfg.K, rs, offsets, wd["w_up"], wd["w_down_t"], flags=f, zero_count=zc)
                M.moe_experts(x, 1, None, one, wd["w_up_shared"][None], wd["w_down_shared_t"][None],
                              flags=f, zero_count=zs)
            torch.cuda.synchronize()
            c = counts.cpu()
            touched = int((c > 0).sum().item())
            blocks = int(((c + ITEM_ROWS - 1) // ITEM_ROWS).sum().item())
            blocks_s = (T + ITEM_ROWS - 1) // ITEM_ROWS
            z_r, sk_r = zc.tolist()
            z_s, sk_s = zs.tolist()
            row = cfg.d * wb
            # FP8: the per-output-channel scales of the touched experts too;
            # MXFP4: their block scales (one byte per 32 weights)
            sc_b = (touched * (cfg.F + cfg.d) + cfg.F_shared + cfg.d) * 4 if fp8 else 0
            if fp4:
                sc_b = 2 * (touched * cfg.F + cfg.F_shared) * cfg.d // 32
            up_b = touched * cfg.F * row + cfg.F_shared * row
            dn_b = (blocks * cfg.F - sk_r) * row + (blocks_s * cfg.F_shared - sk_s) * row
            router_b = cfg.E * cfg.d * 4
            need += up_b + dn_b + router_b + sc_b
            dense += up_b + touched * cfg.F * row + cfg.F_shared * row + router_b + sc_b
            zeros += z_r
            elems += T * cfg.K * cfg.F
            skipped += sk_r
            rows += blocks * cfg.F
        need /= ncopy
        dense /= ncopy
        gbps = need / (us * 1e-6) / 1e9
        out[str(T)] = {"us_per_step": us, "us_per_step_eager": us_eager, "graph_replay_matches_eager": graph_ok,
                       "tokens_per_s": T / (us * 1e-6),
                       "weight_bytes_read": need, "GBps_read": gbps,
                       "hbm_frac": gbps / HBM_PEAK_GBPS,
                       "GBps_dense_equivalent": dense / (us * 1e-6) / 1e9,
                       "zero_frac_routed": zeros / elems, "skipped_row_frac_routed": skipped / rows}
        log(f"[bench] decode{' ' + fmt if fmt else ''} T={T}: {us:.1f} us/step, {gbps:.0f} GB/s read "
            f"({gbps / HBM_PEAK_GBPS:.1%}), zeros {zeros / elems:.3f}")
    return out


def prenorm_residual(args, M, synth, torch, cfg, x, wd, base_ms):
    """The same layer with the fused front and back (RMSNorm in front, the
    residual behind): its step time, and the RMSNorm kernel's own time and
    HBM rate (it reads x and writes the normalised rows once)."""
    wdn = dict(wd, w_norm=synth.make_norm_weight(cfg).cuda())
    p = dict(cfg.params(), prenorm_residual=1, norm_eps=cfg.norm_eps, act_dtype=cfg.dtype)
    desc = M.make_desc(p, M.MOE_BF16)
    wst = M.make_weights_struct(wdn)
    ws = torch.empty(M.moe_workspace_size(desc, cfg.T), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda")
    warm_up(lambda: M.moe_layer_forward(desc, wst, x, out=out, ws=ws), args, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        M.moe_layer_forward(desc, wst, x, out=out, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # the RMSNorm kernel alone: 20 launches captured in a HIP graph and
    # replayed, so the host's per-call cost does not space them out (in
    # stage events the first stage of a call also carries its launch latency)
    xn = torch.empty_like(x)
    M.moe_rmsnorm(x, wdn["w_norm"], cfg.norm_eps, out=xn)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(20):
            M.moe_rmsnorm(x, wdn["w_norm"], cfg.norm_eps, out=xn)
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    norm_ms = e0.elapsed_time(e1) / 100
    del g
    norm_bytes = 2 * cfg.T * cfg.d * 2 + cfg.d * 2
    gbps = norm_bytes / (norm_ms * 1e-3) / 1e9
    log(f"[bench] {cfg.name} with RMSNorm front and residual: {ms:.4f} ms/step, norm {norm_ms * 1e3:.1f} us "
        f"({gbps:.0f} GB/s)")
    return {"ms_per_step": ms, "tokens_per_s": cfg.T / (ms * 1e-3), "extra_ms_over_plain": ms - base_ms,
            "norm_us": norm_ms * 1e3, "norm_bytes": norm_bytes, "norm_GBps": gbps,
            "norm_hbm_frac": gbps / HBM_PEAK_GBPS, "norm_eps": cfg.norm_eps}


def capacity_variant(args, M, synth, torch, cfg, x, wd, base_ms, cf=1.0):
    """The same layer with a fixed capacity per expert (capacity factor cf):
    its step time, the dispatch stage (dropless dispatch + arbitration +
    tile plans) and how many routes overflowed."""
    p = dict(cfg.params(), capacity_factor=cf)
    desc = M.make_desc(p, M.MOE_BF16)
    wst = M.make_weights_struct(wd)
    ws = torch.empty(M.moe_workspace_size(desc, cfg.T), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda")
    warm_up(lambda: M.moe_layer_forward(desc, wst, x, out=out, ws=ws), args, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        M.moe_layer_forward(desc, wst, x, out=out, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nst = len(M.STAGES)
    ev = HipEvents(2 * nst)
    disp = 0.0
    for _ in range(args.steps):
        M.moe_layer_forward(desc, wst, x, out=out, ws=ws, events=ev.array)
        torch.cuda.synchronize()
        i = M.STAGES.index("dispatch")
        disp += ev.elapsed_ms(2 * i, 2 * i + 1) / args.steps
    ev.close()
    C = M.moe_capacity_slots(cfg.T, cfg.K, cfg.E, cf)
    z = M.moe_router_logits(x, wd["w_router"])
    ids, w = M.moe_route(z, wd["bias"], cfg.K, cfg.n_group, cfg.topk_group, cfg.norm_topk_prob,
                         cfg.routed_scaling_factor)
    counts, offsets, _, _ = M.moe_dispatch_capacity(ids, w, cfg.E, C)
    kept = int(offsets[-1].item())
    log(f"[bench] {cfg.name} with capacity factor {cf} (C={C}): {ms:.4f} ms/step, "
        f"{cfg.T * cfg.K - kept} of {cfg.T * cfg.K} routes overflowed")
    return {"capacity_factor": cf, "slots_per_expert": C, "ms_per_step": ms,
            "tokens_per_s": cfg.T / (ms * 1e-3), "ms_vs_dropless": ms - base_ms,
            "dispatch_stage_us": disp * 1e3, "routes": cfg.T * cfg.K, "routes_kept": kept}


def lowp_experts(args, M, synth, torch, cfg, w_cpu, x, base_ms, fmt="fp8"):
    """The layer with low-precision expert weights and bf16 activations:
    fmt "fp8" (E4M3, an fp32 scale per output channel, W8A16) or "mxfp4"
    (E2M1, an E8M0 scale per 32 inputs, W4A16): the prefill step, its
    expert GEMM stages, and the decode batches (graph-replayed,
    zero-skipping)."""
    wd8 = M.device_weights(w_cpu, "cuda", expert_dtype=fmt)
    cfg8 = synth.dataclasses.replace(cfg, expert_dtype=fmt)
    desc = M.make_desc(cfg8.params(), M.MOE_BF16)
    wst = M.make_weights_struct(wd8)
    ws = torch.empty(M.moe_workspace_size(desc, cfg.T), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda")
    warm_up(lambda: M.moe_layer_forward(desc, wst, x, out=out, ws=ws), args, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        M.moe_layer_forward(desc, wst, x, out=out, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nst = len(M.STAGES)
    ev = HipEvents(2 * nst)
    stage_ms = [0.0] * nst
    for _ in range(args.steps):
        M.moe_layer_forward(desc, wst, x, out=out, ws=ws, events=ev.array)
        torch.cuda.synchronize()
        for s in range(nst):
            stage_ms[s] += ev.elapsed_ms(2 * s, 2 * s + 1) / args.steps
    ev.close()
    st = dict(zip(M.STAGES, stage_ms))
    counts, _, _ = routing_counts(M, x, wd8, cfg)
    touched = int((counts > 0).sum().item())
    n_w = 2 * (touched * cfg.F * cfg.d + cfg.F_shared * cfg.d)
    w8_bytes = n_w // 2 + n_w // 32 if fmt in ("mxfp4", "mxfp4_a8") else n_w
    log(f"[bench] {cfg.name} with {fmt} experts: {ms:.4f} ms/step (up {st['up']:.4f}, down {st['down']:.4f} ms)")
    fmt_doc = {"fp8": "E4M3 (OCP FN) weights, fp32 scale per output channel, bf16 activations",
               "mxfp4": "MXFP4 (OCP MX E2M1) weights, E8M0 scale per 32 inputs, bf16 activations",
               "mxfp4_a8": "MXFP4 weights and MXFP8 (OCP MX E4M3) inputs of both expert products on the "
                           "block-scaled MFMA (W4A8)"}
    res = {"format": fmt_doc[fmt],
           "prefill": {"ms_per_step": ms, "tokens_per_s": cfg.T / (ms * 1e-3), "ms_vs_bf16": ms - base_ms,
                       "stages_ms": {k: round(v, 5) for k, v in st.items()},
                       "expert_weight_bytes": w8_bytes}}
    # the expert GEMMs against the roofline: FLOPs at the FP8 MFMA peak (the
    # rate of the FP8 x FP4 block-scaled MFMA), algorithmic bytes = the
    # touched experts' codes and scales (and the x rows for the up product)
    R = cfg.T * cfg.K
    fl = 2.0 * R * cfg.d * cfg.F + 2.0 * cfg.T * cfg.d * cfg.F_shared
    for stage in ("up", "down"):
        t = st[stage] * 1e-3
        by = w8_bytes // 2 + (cfg.T * cfg.d * 2 if stage == "up" else 0)
        res["prefill"][f"{stage}_tflops"] = fl / t / 1e12
        res["prefill"][f"{stage}_GBps"] = by / t / 1e9
        if fmt == "mxfp4_a8":
            res["prefill"][f"{stage}_fp8_mfma_frac"] = fl / t / 1e12 / FP8_PEAK_TFLOPS
        else:
            res["prefill"][f"{stage}_bf16_mfma_frac"] = fl / t / 1e12 / BF16_PEAK_TFLOPS
    if not args.no_decode and fmt != "mxfp4_a8":
        res["decode"] = decode(args, M, synth, torch, w_cpu, wd8, fmt=fmt)
    del wd8
    torch.cuda.empty_cache()
    return res


def backward_pass(args, M, synth, torch, cfg, w_cpu, x, wd, fwd_ms):
    """The layer's backward (f3) on the same batch, given a seeded synthetic
    upstream gradient dY ~ N(0, 1) in bf16: step time, per-phase times (HIP
    events around each phase inside the call) and the dominant GEMM phase
    against the bf16 MFMA peak."""
    wb = M.device_weights_bwd(w_cpu, "cuda")
    gen = torch.Generator().manual_seed(7)
    dy = torch.randn(cfg.T, cfg.d, generator=gen).to(torch.bfloat16).cuda()
    desc = M.make_desc(cfg.params(), M.MOE_BF16)
    wst = M.make_weights_struct(wd)
    ws = torch.empty(M.moe_backward_workspace_size(desc, cfg.T), dtype=torch.uint8, device="cuda")
    grads = M.moe_layer_backward(desc, wst, wb, x, dy, ws=ws)
    warm_up(lambda: M.moe_layer_backward(desc, wst, wb, x, dy, grads=grads, ws=ws), args, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    steps = max(1, args.steps // 2)
    e0.record()
    for _ in range(steps):
        M.moe_layer_backward(desc, wst, wb, x, dy, grads=grads, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # the training step: the forward that keeps its state, then the backward
    # that reuses it
    out = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda")
    for _ in range(2):
        M.moe_layer_forward_train(desc, wst, x, ws, out=out)
        M.moe_layer_backward(desc, wst, wb, x, dy, grads=grads, ws=ws, saved=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        M.moe_layer_forward_train(desc, wst, x, ws, out=out)
        M.moe_layer_backward(desc, wst, wb, x, dy, grads=grads, ws=ws, saved=True)
    e1.record()
    torch.cuda.synchronize()
    train_ms = e0.elapsed_time(e1) / steps
    nst = len(M.BWD_STAGES)
    ev = HipEvents(2 * nst)
    st = [0.0] * nst
    for _ in range(steps):
        M.moe_layer_backward(desc, wst, wb, x, dy, grads=grads, ws=ws, events=ev.array)
        torch.cuda.synchronize()
        for i in range(nst):
            st[i] += ev.elapsed_ms(2 * i, 2 * i + 1) / steps
    ev.close()
    st = dict(zip(M.BWD_STAGES, st))
    R, T, d, F, Fs, L = cfg.T * cfg.K, cfg.T, cfg.d, cfg.F, cfg.F_shared, cfg.d_latent
    de = L or d  # the experts' input width
    one = 2.0 * R * de * F + 2.0 * T * d * Fs  # one routed + shared product pass
    lat = 2.0 * T * d * L  # one latent projection (0 without)
    # the forward: both expert products and both projections; the backward
    # phases: dy_lat (gates), dx_lat W_lin (dx), dW_lout (dw_down), dW_lin (dw_up)
    flops = {"forward": 2 * one + 2 * lat, "gates": lat, "dh": one, "dx": one + lat, "dw_down": one + lat,
             "dw_up": one + lat}
    counts, _, _ = routing_counts(M, x, wd, cfg)
    touched = int((counts > 0).sum().item())
    Rp = R + 7 * cfg.E
    # algorithmic bytes of the weight-gradient phases: the transposed operands
    # read once, the fp32 gradients written once
    lb = T * (d + L) * 2 + d * L * 4 if L else 0
    wbytes = {"dw_down": Rp * (de + F) * 2 + T * (d + Fs) * 2 + (touched * de * F + d * Fs) * 4 + lb,
              "dw_up": Rp * (F + de) * 2 + T * (Fs + d) * 2 + (touched * F * de + Fs * d) * 4 + lb,
              "dh": touched * de * F * 2 + d * Fs * 2 + R * de * 2 + T * d * 2 + (R * F + T * Fs) * 2 * 2,
              "dx": touched * F * de * 2 + Fs * d * 2 + (R * F + T * Fs) * 2 + R * de * 4 + T * d * 4}
    dom = max(("dh", "dx", "dw_down", "dw_up"), key=lambda k: st[k])
    tf = flops[dom] / (st[dom] * 1e-3) / 1e12
    total_flops = sum(flops.values())
    log(f"[bench] {cfg.name} backward: {ms:.4f} ms/step ({', '.join(f'{k} {v:.3f}' for k, v in st.items())}); "
        f"training step (forward + saved backward) {train_ms:.4f} ms")
    return {"ms_per_step": ms, "tokens_per_s": cfg.T / (ms * 1e-3),
            "train_step_ms": train_ms, "train_tokens_per_s": cfg.T / (train_ms * 1e-3),
            "train_step": "moe_layer_forward_train + moe_layer_backward_saved (the backward reuses the forward's state)",
            "stages_ms": {k: round(v, 5) for k, v in st.items()},
            "gflop": total_flops / 1e9, "tflops": total_flops / (ms * 1e-3) / 1e12,
            "mfma_frac": total_flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "dominant": {"stage": dom, "tflops": tf, "mfma_frac": tf / BF16_PEAK_TFLOPS,
                         "algorithmic_bytes": wbytes[dom],
                         "hbm_gbps": wbytes[dom] / (st[dom] * 1e-3) / 1e9,
                         "hbm_frac": wbytes[dom] / (st[dom] * 1e-3) / 1e9 / HBM_PEAK_GBPS},
            "dy": "seeded N(0, 1) in bf16; the forward is recomputed inside the call"}


def ep_share(args, M, synth, torch, cfg, x, wd, P=8):
    """One GPU's share of an expert-parallel layer over P GPUs, which this
    build does not run (one GPU): moe_experts on the first E / P experts and
    the routes the batch sends them, at their real shape.  The exchange of
    rows between GPUs, the router, the shared expert and the combine are
    left out.  Informative, beside the headline."""
    counts, offsets, rs = routing_counts(M, x, wd, cfg)
    E_loc = cfg.E // P
    off = offsets[: E_loc + 1].contiguous()
    n_rows = int(off[-1].item())
    w_up = wd["w_up"][:E_loc]
    w_dn = wd["w_down_t"][:E_loc]
    y = torch.empty((cfg.T * cfg.K, cfg.d), dtype=torch.bfloat16, device="cuda")
    need = M.lib().moe_experts_workspace_size(M.MOE_BF16, cfg.T, cfg.d, cfg.K, E_loc, cfg.F, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def step():
        M.moe_experts(x, cfg.K, rs, off, w_up, w_dn, y_packed=y, ws=ws)

    warm_up(step, args, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    touched = int((counts[:E_loc] > 0).sum().item())
    src = (rs[:n_rows] // cfg.K).cpu()
    tokens = int(torch.unique(src).numel())
    flops = 4.0 * n_rows * cfg.d * cfg.F
    by = touched * 2 * cfg.F * cfg.d * 2 + tokens * cfg.d * 2 + n_rows * cfg.d * 2
    t = ms * 1e-3
    log(f"[bench] expert-parallel share (E/{P} = {E_loc} experts, {n_rows} routes): {ms:.4f} ms, "
        f"{by / t / 1e9:.0f} GB/s, {flops / t / 1e12:.0f} TFLOP/s")
    return {"what": f"moe_experts on experts 0..{E_loc - 1} of {cfg.E} and the {n_rows} routes the "
                    f"{cfg.name} batch sends them (one GPU of {P}; no exchange, router, shared expert or combine)",
            "experts": E_loc, "routes": n_rows, "ms": ms, "routes_per_s": n_rows / t,
            "tflops": flops / t / 1e12, "mfma_frac": flops / t / 1e12 / BF16_PEAK_TFLOPS,
            "algorithmic_bytes": by, "GBps": by / t / 1e9, "hbm_frac": by / t / 1e9 / HBM_PEAK_GBPS}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _time_oracle(fn, T, budget_s, min_reps=1):
    """Calls fn() (one pass over T tokens) until budget_s seconds have
    passed (at least min_reps times); returns (tokens/s, passes, seconds)."""
    reps = 0
    t0 = time.perf_counter()
    while True:
        fn()
        reps += 1
        t = time.perf_counter() - t0
        if reps >= min_reps and t >= budget_s:
            break
        if reps >= min_reps and t * (reps + 1) / reps > 2.0 * budget_s:
            break
    return reps * T / t, reps, t


def cpu_baseline(args, cfg, w_cpu, x_cpu, torch, more=None):
    """The oracle as it stands (numpy float64, expert-major), on the host
    cores, on bounded samples of the workloads; conversion to float64 is
    outside the timed region.  The headline object is the Nano prefill
    batch with all BLAS threads; ``per_config`` adds the same with one
    thread, each decode batch, the latent and stress layers (``more``:
    {name: (cfg, w_cpu, x_cpu)}) and the tiny fp32 layer with the loop-only
    token-major oracle beside it."""
    import numpy as np
    import threadpoolctl

    import oracle.moe_oracle as O
    from routed_relu_expert_amd import synth
    log("[bench] cpu baseline: converting weights to float64 (untimed)")
    w64 = {k: synth.to_f64(v) for k, v in w_cpu.items()}
    x64 = synth.to_f64(x_cpu)
    p = cfg.params()
    info = threadpoolctl.threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    model = _cpu_model()
    # size the sample to about cpu_seconds: a prefix of the batch when one
    # pass over it would take longer, else whole-batch repetitions (the
    # probe is large enough that the per-expert fixed cost does not dominate)
    Ts = min(512, cfg.T)
    t0 = time.perf_counter()
    O.layer_forward(p, x64[:Ts], w64)
    t1 = time.perf_counter() - t0
    if t1 * cfg.T / Ts <= args.cpu_seconds:
        Ts2 = cfg.T
    else:
        Ts2 = int(min(cfg.T, max(Ts, Ts * args.cpu_seconds / max(t1, 1e-3))))
    reps, tokens = 0, 0
    t0 = time.perf_counter()
    while True:
        O.layer_forward(p, x64[:Ts2], w64)
        reps += 1
        tokens += Ts2
        t2 = time.perf_counter() - t0
        if t2 >= 0.66 * args.cpu_seconds or Ts2 < cfg.T:
            break
    log(f"[bench] cpu baseline: {reps} x {Ts2} tokens in {t2:.2f} s on {cores} threads ({model})")
    res = {"value": tokens / t2, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu_model": model,
           "sample": f"{reps} pass(es) over the first {Ts2} of the {cfg.T} tokens of the {cfg.name} "
                     f"batch with all {cfg.E} experts' weights, numpy float64 expert-major oracle, "
                     f"{t2:.1f} s"}
    if args.cpu_brief:
        return res
    per = {}
    budget = args.cpu_seconds / 3
    # one BLAS thread, a prefix of the same batch
    with threadpoolctl.threadpool_limits(1, user_api="blas"):
        Ts1 = 256
        v, n, t = _time_oracle(lambda: O.layer_forward(p, x64[:Ts1], w64), Ts1, budget)
    per["nano_prefill_1_thread"] = {"tokens_per_s": v, "threads": 1, "sample": f"{n} x first {Ts1} tokens, {t:.1f} s"}
    log(f"[bench] cpu baseline nano_prefill, 1 thread: {v:.0f} tokens/s")
    # decode batches: the same weights, x from the decode stream
    xd = synth.to_f64(synth.make_inputs(synth.NANO_DECODE, w_cpu)["x"])
    for T in synth.DECODE_T:
        v, n, t = _time_oracle(lambda: O.layer_forward(p, xd[:T], w64), T, budget / 4, min_reps=2)
        per[f"nano_decode_T{T}"] = {"tokens_per_s": v, "threads": cores, "sample": f"{n} passes, {t:.1f} s"}
        log(f"[bench] cpu baseline nano_decode T={T}: {v:.1f} tokens/s")
    del w64
    for name, (c2, w2, x2) in (more or {}).items():
        log(f"[bench] cpu baseline {name}: converting weights to float64 (untimed)")
        w2_64 = {k: synth.to_f64(v) for k, v in w2.items()}
        x2_64 = synth.to_f64(x2)
        Tn = min(c2.T, args.cpu_other_rows)
        v, n, t = _time_oracle(lambda: O.layer_forward(c2.params(), x2_64[:Tn], w2_64), Tn, budget)
        per[name] = {"tokens_per_s": v, "threads": cores,
                     "sample": f"{n} pass(es) over the first {Tn} of the {c2.T} tokens, {t:.1f} s"}
        log(f"[bench] cpu baseline {name}: {v:.0f} tokens/s")
        del w2_64, x2_64
    # the tiny fp32 layer: expert-major and the loop-only token-major oracle
    tc = synth.TINY_F32
    wt = synth.make_weights(tc)
    wt64 = {k: synth.to_f64(v) for k, v in wt.items()}
    xt64 = synth.to_f64(synth.make_inputs(tc, wt)["x"])
    v, n, t = _time_oracle(lambda: O.layer_forward(tc.params(), xt64, wt64), tc.T, 1.0, min_reps=3)
    v2, n2, t2 = _time_oracle(lambda: O.token_major_forward(tc.params(), xt64, wt64), tc.T, 1.0, min_reps=2)
    per["tiny_f32"] = {"tokens_per_s": v, "token_major_loop_tokens_per_s": v2, "threads": cores,
                       "sample": f"{n} / {n2} passes over the {tc.T} tokens"}
    res["per_config"] = per
    return res


def other_config(args, M, synth, torch, cfg, w=None):
    """A leg beside the headline: the layer of another configuration -- the
    latent layer or the skewed stress batch -- timed as the headline is,
    with each stage's algorithmic work against the roofline (the latent
    projections run only here).  ``w``: the config's CPU weights when
    already drawn (the stress batch reuses the prefill weights).  Returns
    the result, the CPU weights (stress bias included) and the CPU input."""
    if w is None:
        log(f"[bench] {cfg.name}: generating weights (seeded)")
        w = synth.make_weights(cfg)
    else:
        w = dict(w)
    inp = synth.make_inputs(cfg, w)
    if "bias" in inp:
        w["bias"] = inp["bias"]
    wd = M.device_weights(w, "cuda")
    x = inp["x"].cuda()
    desc = M.make_desc(cfg.params(), M.MOE_BF16)
    wst = M.make_weights_struct(wd)
    ws = torch.empty(M.moe_workspace_size(desc, cfg.T), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda")
    settled = warm_up(lambda: M.moe_layer_forward(desc, wst, x, out=out, ws=ws), args, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        M.moe_layer_forward(desc, wst, x, out=out, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nst = len(M.STAGES)
    ev = HipEvents(2 * nst)
    stage_ms = [0.0] * nst
    for _ in range(args.steps):
        M.moe_layer_forward(desc, wst, x, out=out, ws=ws, events=ev.array)
        torch.cuda.synchronize()
        for i in range(nst):
            stage_ms[i] += ev.elapsed_ms(2 * i, 2 * i + 1) / args.steps
    ev.close()
    st = dict(zip(M.STAGES, stage_ms))
    counts, _, _ = routing_counts(M, x, wd, cfg)
    touched = int((counts > 0).sum().item())
    T, d, L, F, Fs, R = cfg.T, cfg.d, cfg.d_latent, cfg.F, cfg.F_shared, cfg.T * cfg.K
    de = cfg.d_e
    work = {  # stage: (flops, algorithmic bytes)
        "router_gemm": (2.0 * T * d * cfg.E, cfg.E * d * 4 + T * d * 2 + T * cfg.E * 4),
        "up": (2.0 * R * de * F + 2.0 * T * d * Fs, touched * F * de * 2 + Fs * d * 2 + T * de * 2 + T * d * 2),
        "down": (2.0 * R * F * de + 2.0 * T * Fs * d, touched * F * de * 2 + Fs * d * 2),
    }
    if L:
        work["latent_in"] = (2.0 * T * d * L, L * d * 2 + T * d * 2 + T * L * 2)
        work["latent_out"] = (2.0 * T * L * d, d * L * 2 + T * L * 2 + T * d * 4 + T * d * 2)
    stages = {}
    for k, (fl, by) in work.items():
        t = st[k] * 1e-3
        stages[k] = {"ms": st[k], "tflops": fl / t / 1e12, "mfma_frac": fl / t / 1e12 / BF16_PEAK_TFLOPS,
                     "GBps": by / t / 1e9, "hbm_frac": by / t / 1e9 / HBM_PEAK_GBPS,
                     "algorithmic_bytes": by, "flops": fl}
    log(f"[bench] {cfg.name}: {ms:.4f} ms/step, {T / (ms * 1e-3) / 1e6:.3f} M tokens/s; " +
        ", ".join(f"{k} {v['ms']:.4f} ms ({v['hbm_frac']:.0%} HBM, {v['mfma_frac']:.0%} MFMA)"
                  for k, v in stages.items()))
    layer_fl = sum(v[0] for v in work.values())
    # algorithmic bytes of the layer: each touched expert's two matrices, the
    # shared expert's, the router and the latent projections read once, x
    # read once and out written once
    layer_by = 2 * touched * F * de * 2 + 2 * Fs * d * 2 + cfg.E * d * 4 + 2 * T * d * 2 + (2 * L * d * 2 if L else 0)
    t = ms * 1e-3
    roof = max(layer_fl / (BF16_PEAK_TFLOPS * 1e12), layer_by / (HBM_PEAK_GBPS * 1e9))
    res = {"workload": cfg.name, "T": T, "d": d, "d_latent": L, "E": cfg.E, "K": cfg.K, "F": F, "F_shared": Fs,
           "n_group": cfg.n_group, "topk_group": cfg.topk_group, "ms_per_step": ms, "warmup_settle": settled,
           "tokens_per_s": T / t, "stages_ms": {k: round(v, 5) for k, v in st.items()},
           "layer": {"gflop": layer_fl / 1e9, "algorithmic_gb": layer_by / 1e9,
                     "mfma_frac": layer_fl / t / 1e12 / BF16_PEAK_TFLOPS,
                     "hbm_frac": layer_by / t / 1e9 / HBM_PEAK_GBPS,
                     "roofline_time_ms": roof * 1e3, "roofline_frac": roof / t},
           "stage_rooflines": stages, "experts_touched": touched,
           "routing": routing_report(counts.cpu().tolist(), T)}
    del wd
    torch.cuda.empty_cache()
    return res, w, inp["x"]


def vendor_gemm(args, torch, cfg, stages):
    """The vendor BLAS (hipBLASLt through torch) on the expert products'
    shapes, for calibration: the routed rows split equally over the experts
    (T K / E each, contiguous, no gather) as one batched product per
    projection, and the shared expert as a plain product.  The layer's own
    grouped GEMMs do more (the gather through the route map, the uneven
    split, the ReLU^2 epilogue) in one launch per projection; their stage
    times are set beside these."""
    E, d, F, Fs, T = cfg.E, cfg.d, cfg.F, cfg.F_shared, cfg.T
    m = cfg.T * cfg.K // E
    g = torch.Generator(device="cuda").manual_seed(5)

    def rnd(*shape):
        return torch.randn(*shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)

    def timed(fn):
        warm_up(fn, args, torch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    out = {"what": f"torch.bmm over {E} experts x {m} rows (equal split) plus the shared expert's torch.matmul, "
                   "bf16, contiguous operands",
           "rows_per_expert": m}
    for proj, (ki, no) in (("up", (d, F)), ("down", (F, d))):
        a, b = rnd(E, m, ki), rnd(E, ki, no)
        ms_r = timed(lambda: torch.bmm(a, b))
        del a, b
        ki_s, no_s = (d, Fs) if proj == "up" else (Fs, d)
        a, b = rnd(T, ki_s), rnd(ki_s, no_s)
        ms_s = timed(lambda: torch.matmul(a, b))
        del a, b
        ours = stages[proj]
        out[proj] = {"routed_ms": ms_r, "shared_ms": ms_s, "vendor_ms": ms_r + ms_s, "layer_gemm_ms": ours,
                     "vendor_over_layer": (ms_r + ms_s) / ours}
        log(f"[bench] vendor BLAS {proj}: routed {ms_r:.4f} ms + shared {ms_s:.4f} ms = {ms_r + ms_s:.4f} ms; "
            f"the layer's grouped GEMM {ours:.4f} ms")
    # a large dense product of the model width: the library's compute-bound rate
    n = 8192
    a, b = rnd(n, d), rnd(d, n)
    ms_d = timed(lambda: torch.matmul(a, b))
    del a, b
    tf = 2.0 * n * n * d / (ms_d * 1e-3) / 1e12
    out["dense"] = {"shape": [n, d, n], "ms": ms_d, "tflops": tf, "mfma_frac": tf / BF16_PEAK_TFLOPS}
    log(f"[bench] vendor BLAS dense {n} x {d} x {n}: {ms_d:.4f} ms, {tf:.0f} TFLOP/s")
    torch.cuda.empty_cache()
    return out


LEGS = ("prenorm", "backward", "capacity", "decode", "fp8", "mxfp4", "w4a8", "ep_share", "vendor_gemm",
        "super_latent", "backward_latent", "nano_stress", "cpu")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-s", type=float, default=1.5,
                    help="warm-up continues until this many seconds have passed (the clock ramps up under load)")
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--decode-T", type=str, default="1,4,16,64")
    ap.add_argument("--decode-marks", action="store_true",
                    help="decode batches eager only, each batch's steps between two spin kernels (for counter traces)")
    ap.add_argument("--legs", type=str, default=",".join(LEGS),
                    help="legs beside the headline prefill step: " + ",".join(LEGS))
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-brief", action="store_true", help="cpu baseline of the headline workload only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-other-rows", type=int, default=512)
    ap.add_argument("--copy-probe-gib", type=float, default=0.0,
                    help="after the timed region, copy this many GiB device-to-device once: the "
                         "plain copy kernel against which rocprofv3 FETCH_SIZE/WRITE_SIZE are scaled")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    args.decode_T = [int(v) for v in args.decode_T.split(",") if v]
    legs = {v for v in args.legs.split(",") if v}
    unknown = legs - set(LEGS)
    if unknown:
        print(f"unknown legs {sorted(unknown)}; known: {','.join(LEGS)}", file=sys.stderr)
        sys.exit(2)
    if args.no_decode:
        legs.discard("decode")
    if args.no_cpu_baseline:
        legs.discard("cpu")
    args.no_decode = "decode" not in legs
    import torch

    import routed_relu_expert_amd as M
    from routed_relu_expert_amd import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    M.lib()
    res, cfg, w_cpu, x_cpu, wd = prefill(args, M, synth, torch)
    x_dev = x_cpu.cuda()
    base = res["ms_per_step"]
    pre = prenorm_residual(args, M, synth, torch, cfg, x_dev, wd, base) if "prenorm" in legs else None
    bwd = backward_pass(args, M, synth, torch, cfg, w_cpu, x_dev, wd, base) if "backward" in legs else None
    cap = capacity_variant(args, M, synth, torch, cfg, x_dev, wd, base) if "capacity" in legs else None
    eps = ep_share(args, M, synth, torch, cfg, x_dev, wd) if "ep_share" in legs else None
    dec = decode(args, M, synth, torch, w_cpu, wd) if "decode" in legs else None
    del wd
    torch.cuda.empty_cache()
    vg = vendor_gemm(args, torch, cfg, res["stages_ms"]) if "vendor_gemm" in legs else None
    f8 = lowp_experts(args, M, synth, torch, cfg, w_cpu, x_dev, base) if "fp8" in legs else None
    f4 = lowp_experts(args, M, synth, torch, cfg, w_cpu, x_dev, base, fmt="mxfp4") if "mxfp4" in legs else None
    w4a8 = lowp_experts(args, M, synth, torch, cfg, w_cpu, x_dev, base, fmt="mxfp4_a8") if "w4a8" in legs else None
    torch.cuda.empty_cache()
    oth, more = [], {}
    if "super_latent" in legs:
        r, w3, x3 = other_config(args, M, synth, torch, synth.SUPER_LATENT)
        oth.append(r)
        more["super_latent"] = (synth.SUPER_LATENT, w3, x3)
    bwd3 = None
    if "backward_latent" in legs:
        # the latent layer's backward (f3) on the super_latent batch
        cfg3 = synth.SUPER_LATENT
        w3, x3 = (more["super_latent"][1], more["super_latent"][2]) if "super_latent" in more else (None, None)
        if w3 is None:
            w3 = synth.make_weights(cfg3)
            inp3 = synth.make_inputs(cfg3, w3)
            if "bias" in inp3:
                w3["bias"] = inp3["bias"]
            x3 = inp3["x"]
        wd3 = M.device_weights(w3, "cuda")
        bwd3 = backward_pass(args, M, synth, torch, cfg3, w3, x3.cuda(), wd3, None)
        del wd3
        torch.cuda.empty_cache()
    if "nano_stress" in legs:
        r, w4, x4 = other_config(args, M, synth, torch, synth.NANO_STRESS, w=w_cpu)
        oth.append(r)
        more["nano_stress"] = (synth.NANO_STRESS, w4, x4)
    cpu = cpu_baseline(args, cfg, w_cpu, x_cpu, torch, more) if "cpu" in legs else None
    line = {
        "metric": "MoE-layer tokens/s + %bf16 MFMA peak (prefill); %HBM BW (decode)",
        "value": res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "nano_prefill_moe_layer", "T": cfg.T, "d": cfg.d, "E": cfg.E,
                   "K": cfg.K, "F": cfg.F, "F_shared": cfg.F_shared, "n_group": cfg.n_group,
                   "topk_group": cfg.topk_group, "routed_scaling_factor": cfg.routed_scaling_factor,
                   "router": "fp32", "seed": cfg.seed},
        "roofline": res["roofline"], "layer": res["layer"], "stages_ms": res["stages_ms"],
        "warmup_settle": res["warmup_settle"],
        "prenorm_residual": pre, "capacity": cap, "decode": dec, "fp8_experts": f8, "mxfp4_experts": f4,
        "w4a8_experts": w4a8, "backward": bwd, "backward_latent": bwd3,
        "ep_share": eps, "vendor_gemm": vg, "other_configs": oth or None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    if args.copy_probe_gib > 0:
        n = int(args.copy_probe_gib * (1 << 30)) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {n * 4} bytes copied device to device")


if __name__ == "__main__":
    main()
