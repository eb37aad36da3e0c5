#!/usr/bin/env python3
"""Throughput of the Stable LatentMoE layer forward on one MI355X.

One step = one full forward of the layer (router logits, quantile cutoffs,
top-k, dispatch, W_down_proj, grouped SiTU-GLU experts, combine + latent
RMSNorm, output projection with the shared experts) over one batch of
synthetic tokens already resident in HBM, through the C ABI (moe_forward).

Prints one JSON line: tokens/s, the roofline of the dominant kernel (timed
with HIP events on its own stream inside the timed loop) and the CPU oracle
timed on a bounded sample of the same workload.

    python bench.py [--config k3_prefill_bf16] [--steps 20] [--warmup 5]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA (the block-scaled MFMA on fp8 operands)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "LatentMoE layer tokens/s; % bf16 MFMA peak (prefill), % HBM BW (decode)"


def phase_work(cfg, touched: int) -> dict:
    """Algorithmic FLOPs and HBM bytes of each phase of one forward.

    Bytes count each operand once: weights actually needed (every touched
    expert once), activations in, results out.  MXFP4 experts count half a
    byte per weight plus one E8M0 byte per 32 weights; the dense weights of
    such a layer are bf16."""
    bt, d, L, E, k = cfg.bt, cfg.d, cfg.latent, cfg.n_experts, cfg.top_k
    I, S, Is = cfg.expert_inter, cfg.n_shared, cfg.shared_inter
    P = bt * k
    ab = 4 if cfg.act == "f32" else 2
    wb = {"f32": 4, "bf16": 2, "fp8": 1, "mxfp4": 2, "mxfp8": 2}[cfg.weight]
    rb = {"f32": 4, "bf16": 2}[cfg.router]
    sc = (lambda r, c: (r // 128) * (c // 128) * 4) if cfg.weight == "fp8" else (lambda r, c: 0)
    if cfg.weight == "mxfp4":
        xw = lambda r, c: r * c // 2 + r * (c // 32)  # an expert matrix, codes + scales
    elif cfg.weight == "mxfp8":
        xw = lambda r, c: r * c + r * (c // 32)
    else:
        xw = lambda r, c: r * c * wb + sc(r, c)
    batch = cfg.cutoff == "batch"
    a8 = getattr(cfg, "act_quant", "none") == "mxfp8"
    # MX FP8 expert inputs: the GEMMs read codes + E8M0 bytes, a quantiser writes them
    qb = (lambda n: n + n // 32) if a8 else (lambda n: n * ab)
    extra = {"xlat_quant": (0, bt * L * ab + bt * L * 33 // 32)} if a8 else {}
    return {**extra,
        "shared_gateup": (2 * bt * d * 2 * S * Is,
                          bt * d * ab + 2 * S * (Is * d * wb + sc(Is, d)) + bt * S * Is * ab),
        "router_logits": (2 * bt * d * E, bt * d * ab + E * d * rb + bt * E * 4 * (2 if batch else 1)),
        "cutoff": (0, bt * E * 4 if batch else 0),
        "topk": (0, bt * E * 4 + P * 8),
        "dispatch": (0, P * 4 + P * 8),
        "down_proj": (2 * bt * d * L, bt * d * ab + L * d * wb + sc(L, d) + bt * L * ab),
        "expert_gateup": (2 * P * 2 * L * I, touched * 2 * xw(I, L) + qb(bt * L) + qb(P * I)),
        "expert_down": (2 * P * L * I, touched * xw(L, I) + qb(P * I) + P * L * ab),
        "combine_norm": (0, P * L * ab + bt * L * ab),
        "output": (2 * bt * (L + S * Is) * d,
                   bt * (L + S * Is) * ab + d * (L + S * Is) * wb + sc(d, L) + S * sc(d, Is)
                   + bt * d * ab),
    }


KERNEL_DIR = "sparse_moe_layer_quantile_amd/csrc"


def kernel_source_hash() -> str:
    """Hash of every HIP source of the layer: counters taken from another
    version of the kernels are not reported."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, KERNEL_DIR)
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(f.encode())
            with open(os.path.join(d, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when it is missing or the kernel sources changed since
    the counters were taken.  Reads are the L2-to-memory read requests
    (TCC_EA0_RDREQ_{32B,64B,128B} x their sizes) when the summary has them, else
    FETCH_SIZE scaled by its reading for a plain copy of known size; writes are
    WRITE_SIZE scaled the same way.  Returns (bytes, method)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None, None
    rec = json.load(open(path))
    k = rec.get("kernels", {}).get(kernel)
    if not k or rec.get("gemm_source_hash") != kernel_source_hash():
        return None, None
    if k.get("ea_read_bytes") is not None:
        return k["ea_read_bytes"] + k["write_bytes"], "TCC_EA0_RDREQ_* bytes + WRITE_SIZE (copy-calibrated)"
    return k["bytes_per_launch"], "FETCH_SIZE + WRITE_SIZE (copy-calibrated)"


def roofline_of(name, flops, nbytes, ms, peak_tflops=PEAK_BF16_TFLOPS):
    t_mfma = flops / (peak_tflops * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        ach = flops / (ms * 1e-3) / 1e12
        out = {"bound": "mfma", "achieved": ach, "peak": peak_tflops, "unit": "TFLOP/s",
               "frac": ach / peak_tflops}
    else:
        ach = nbytes / (ms * 1e-3) / 1e9
        out = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
               "frac": ach / PEAK_HBM_GBS}
    out.update({"traffic": None, "kernel": name, "ms": ms, "algorithmic_flops": flops,
                "algorithmic_bytes": nbytes,
                "mfma_frac": flops / (ms * 1e-3) / (peak_tflops * 1e12),
                "hbm_frac": nbytes / (ms * 1e-3) / (PEAK_HBM_GBS * 1e9)})
    return out


def ffn_phase_work(cfg) -> dict:
    """Algorithmic FLOPs and HBM bytes of each phase of the dense FFN."""
    bt, d, I = cfg.bt, cfg.d, cfg.inter
    ab = 4 if cfg.act == "f32" else 2
    return {
        "ffn_norm": (0, 2 * bt * d * ab + 4 * d),
        "ffn_gateup": (2 * bt * d * 2 * I, bt * d * ab + 2 * I * d * ab + bt * I * ab),
        "ffn_down": (2 * bt * I * d, bt * I * ab + d * I * ab + 2 * bt * d * ab),
    }


def ffn_cpu_baseline(cfg, seed: int, n_rows: int) -> dict:
    """The fp64 CPU oracle on a bounded sample of rows of the same FFN workload."""
    import oracle
    import synth
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    sp = synth.ffn_specs(cfg)
    m = {n: oracle.Mat(synth.ffn_host_tensor(cfg, n, seed).reshape(sp[n].shape))
         for n in ("w_gate", "w_up", "w_down")}
    rows = np.arange(min(n_rows, cfg.bt))
    x = oracle.decode(synth.ffn_host_rows(cfg, "x", rows, seed))
    r = oracle.decode(synth.ffn_host_rows(cfg, "r", rows, seed))
    g = synth.ffn_gamma(cfg)
    shape = oracle.FfnShape(cfg.d, cfg.inter, cfg.beta, cfg.beta_u, cfg.rms_eps)
    t0 = time.perf_counter()
    for i in range(len(rows)):
        oracle.dense_ffn(shape, m["w_gate"], m["w_up"], m["w_down"], x[i], r[i], g)
    dt = time.perf_counter() - t0
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(rows)} of {cfg.bt} rows through RMSNorm, gate/up, SiTU, down and "
                      f"the residual ({dt:.1f} s); extrapolated to tokens/s"}


def bench_ffn(args) -> int:
    """The dense layer-1 FFN workloads: same timing protocol and JSON line."""
    import torch
    import synth
    import sparse_moe_layer_quantile_amd as moe
    cfg = synth.FFN_CONFIGS[args.config]
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    t = synth.ffn_device_layer(cfg, args.seed)
    layer = moe.DenseFFN(moe.make_ffn_config(cfg.d, cfg.inter, cfg.beta, cfg.beta_u,
                                             cfg.rms_eps, act=cfg.act), t)
    x, r = t["x"], t["r"]
    y = torch.empty_like(x)
    moe.profile_enable(True)
    for _ in range(args.warmup):
        layer.forward(x, r, out=y)
    torch.cuda.synchronize()
    moe.profile_read()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        layer.forward(x, r, out=y)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1e3 / args.steps
    phases = {n: v for n, v in moe.profile_read().items() if n.startswith("ffn_")}
    moe.profile_enable(False)
    work = ffn_phase_work(cfg)
    dom = max(phases, key=lambda n: phases[n][0])
    roof = roofline_of(dom, work[dom][0], work[dom][1], phases[dom][0])
    roof["traffic"], roof["traffic_method"] = measured_traffic(cfg.name, dom)
    line = {
        "metric": "dense layer-1 FFN tokens/s; % bf16 MFMA peak (prefill), % HBM BW (decode)",
        "value": cfg.bt * args.steps / dt,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.act == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "bt": cfg.bt, "d": cfg.d, "inter": cfg.inter,
                   "parallelism": "1 GPU"},
        "roofline": roof,
        "layer": {"tflops": cfg.flops() / (ms_step * 1e-3) / 1e12,
                  "mfma_frac": cfg.flops() / (ms_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)},
        "phases_ms": {n: round(v[0], 4) for n, v in phases.items()},
        "kernel_sources": kernel_source_hash(),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = ffn_cpu_baseline(cfg, args.seed, min(args.cpu_tokens, 64))
    print(json.dumps(line), flush=True)
    return 0


def bench_tier(args, cfg) -> int:
    """Low-batch decode with the routed experts in pinned host memory and an HBM
    cache of cfg.tier_slots experts (moe_tier_*).  Each step is one forward of a
    new token batch (a pool of 16 seeded batches), with the cache's plan and
    observe calls around it, and ends with the host waiting for the step's
    output, as an autoregressive decode loop does before its next step; the
    cache warms during 4 x warmup steps.  Reported beside it: the same steps
    with every expert resident in HBM, and with none cached (every expert read
    over PCIe)."""
    import torch
    import sparse_moe_layer_quantile_amd as moe
    import synth

    torch.cuda.set_device(0)
    layer, _ = device_layer(cfg, args.seed)
    pool = [synth.device_layer(cfg, seed=1000 + i, names=["x"])["x"] for i in range(16)]
    mx = cfg.weight != "bf16"
    names = ["w_gate", "w_up", "w_down"] + (["e8_gate", "e8_up", "e8_down"] if mx else [])
    host = {n: layer.tensors[n].cpu().pin_memory() for n in names}
    host_bytes = sum(t.numel() * t.element_size() for t in host.values())
    E, P = cfg.n_experts, cfg.bt * cfg.top_k
    bufs = dict(counts=torch.empty(E, dtype=torch.int32, device="cuda"),
                offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
                perm=torch.empty(P, dtype=torch.int32, device="cuda"),
                inv_perm=torch.empty(P, dtype=torch.int32, device="cuda"))
    y = torch.empty((cfg.bt, cfg.d), dtype=torch.bfloat16, device="cuda")

    def run(step_fn, warm, steps):
        for i in range(warm):
            step_fn(pool[i % len(pool)])
            torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step_fn(pool[(warm + i) % len(pool)])
            torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    ms_resident = run(lambda x: layer.forward(x, out=y), args.warmup, args.steps)
    copy = torch.cuda.Stream()
    out = {}
    for n_slots in (0, cfg.tier_slots):
        tier = moe.ExpertTier(layer.cfg, host, n_slots, decay=0.9, max_loads=32)
        t = {n: v for n, v in layer.tensors.items() if n not in names}
        t["expert_tab"] = tier.table
        tl = moe.StableLatentMoE(layer.cfg, t)

        def step(x):
            tier.plan(copy)
            tl.forward(x, out=y, dispatch=bufs)
            tier.observe(bufs["counts"])

        warm = 4 * args.warmup if n_slots else args.warmup
        for i in range(warm):
            step(pool[i % len(pool)])
            torch.cuda.synchronize()
        s0 = tier.stats()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(pool[(warm + i) % len(pool)])
            torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        for _ in range(2):  # fold the timed steps' last counts
            tier.plan(copy)
            torch.cuda.synchronize()
        s1 = tier.stats()
        d = {k: s1[k] - s0[k] for k in s1}
        out[n_slots] = dict(ms=ms, hbm_pair_frac=d["pairs_hbm"] / max(d["pairs"], 1),
                            loads_per_step=d["loads"] / args.steps,
                            bytes_loaded_per_step=d["bytes_loaded"] / args.steps,
                            resident=s1["resident"])
        tier.close()
        del tl, tier
    tiered = out[cfg.tier_slots]
    line = {
        "metric": "tiered-expert decode tokens/s (experts in host DRAM, HBM cache)",
        "value": cfg.bt / (tiered["ms"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": tiered["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "bt": cfg.bt, "d": cfg.d, "latent": cfg.latent,
                   "n_experts": cfg.n_experts, "top_k": cfg.top_k,
                   "expert_inter": cfg.expert_inter, "weights": cfg.weight,
                   "router_bias": cfg.bias, "cutoff": cfg.cutoff, "parallelism": "1 GPU"},
        "tiering": {"cache_slots": cfg.tier_slots,
                    "cache_bytes": cfg.tier_slots * moe.tier_slot_bytes(layer.cfg),
                    "host_expert_bytes": host_bytes,
                    "tiered": tiered, "host_only": out[0],
                    "all_resident_ms": ms_resident},
        "roofline": None,
        "kernel_sources": kernel_source_hash(),
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline(cfg, seed: int, n_tokens: int, logits=None, threads=None) -> dict:
    """The fp64 CPU oracle on a bounded sample of the same workload: on the
    host's cores (OMP_NUM_THREADS) or on `threads` of them.  The batch
    quantile runs on this batch's logits when given (else on a matrix of the
    same shape)."""
    import oracle
    import synth
    saved = oracle.get_threads()
    if threads is not None:
        oracle.set_threads(threads)
    try:
        out = _cpu_baseline(cfg, seed, n_tokens, logits)
    finally:
        oracle.set_threads(saved)
    return out


def _cpu_baseline(cfg, seed, n_tokens, logits):
    import oracle
    import synth
    cores = oracle.get_threads()
    n_params = sum(sp.numel for n, sp in synth.specs(cfg).items() if n != "x")
    if n_params <= 2e8:  # small layers: the whole oracle forward (weights held as fp64)
        lay = synth.host_layer(cfg, seed)
        t0 = time.perf_counter()
        oracle.forward(cfg, lay, cutoff=oracle.BATCH if cfg.cutoff == "batch" else oracle.GIVEN)
        dt = time.perf_counter() - t0
        return {"value": cfg.bt / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
                "sample": f"whole forward of all {cfg.bt} tokens ({dt:.1f} s)"}
    rng = np.random.default_rng(seed)
    tokens = np.sort(rng.choice(cfg.bt, size=min(n_tokens, cfg.bt), replace=False))
    sp = synth.specs(cfg)
    mats = {n: synth.host_tensor(cfg, n, seed).reshape(sp[n].shape)
            for n in ("w_router", "w_down_proj", "w_up_proj", "sh_gate", "sh_up", "sh_down")}
    for n in ("w_down_proj", "w_up_proj", "sh_gate", "sh_up", "sh_down"):
        s = synth.host_scales(cfg, n, seed)
        if s is not None:
            mats["scale:" + n] = s
    mats["router_bias"] = synth.router_bias(cfg)
    mats["gamma"] = synth.gamma(cfg)
    w = oracle.Weights(mats)
    xrows = synth.host_rows(cfg, "x", tokens, seed)
    timed = 0.0
    # router logits + top-k of the sample
    t0 = time.perf_counter()
    z64 = oracle.router_logits(cfg, w, xrows)
    z32 = z64.astype(np.float32)
    timed += time.perf_counter() - t0
    # batch quantile over a full-size logit matrix, amortised over the batch
    q = 0.0
    if cfg.cutoff == "batch":
        zfull = (np.ascontiguousarray(logits, np.float32) if logits is not None else
                 rng.standard_normal((cfg.bt, cfg.n_experts), dtype=np.float32))
        t0 = time.perf_counter()
        alpha = oracle.quantile(zfull, cfg.quantile_rank)
        q = time.perf_counter() - t0
        del zfull
    else:
        alpha = np.zeros(cfg.n_experts, np.float32)
    t0 = time.perf_counter()
    idx, wts = oracle.topk(z32, cfg.top_k, alpha=alpha, z64=z64)
    xd = oracle.decode(xrows)
    xlat = np.stack([oracle.matvec(w.mats["w_down_proj"], xd[i]) for i in range(len(tokens))])
    timed += time.perf_counter() - t0
    # experts, expert-major; regenerating an expert's matrices is not timed
    o = np.zeros((len(tokens), cfg.top_k, cfg.latent))
    by_e = {}
    for i in range(len(tokens)):
        for j in range(cfg.top_k):
            by_e.setdefault(int(idx[i, j]), []).append((i, j))
    esc = {n: synth.host_scales(cfg, n, seed) for n in ("w_gate", "w_up", "w_down")}
    for e, pairs in by_e.items():
        g, u, dn = (oracle.Mat(synth.host_matrix(cfg, n, e, seed),
                               None if esc[n] is None else esc[n][e])
                    for n in ("w_gate", "w_up", "w_down"))
        t0 = time.perf_counter()
        for i, j in pairs:
            o[i, j] = oracle.expert(cfg, g, u, dn, xlat[i])
        timed += time.perf_counter() - t0
    t0 = time.perf_counter()
    for i in range(len(tokens)):
        _, n = oracle.combine_norm(cfg, o[i], wts[i], mats["gamma"])
        oracle.output(cfg, w, n, xd[i])
    timed += time.perf_counter() - t0
    per_token = timed / len(tokens) + q / cfg.bt
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"{len(tokens)} of {cfg.bt} tokens through router logits, top-k, "
                       f"W_down, {cfg.top_k} experts, combine+RMSNorm, W_up and shared "
                       f"experts ({timed:.1f} s), plus the batch quantile over the "
                       f"{cfg.bt}x{cfg.n_experts} logits of the batch ({q:.2f} s) amortised "
                       f"per token; extrapolated to tokens/s")}


def backward_flops(cfg) -> float:
    """Multiply-adds x 2 of one backward call: the recomputed forward GEMMs
    (x_lat, the experts' gate / up / down, the shared gate / up) and the
    gradient GEMMs (two per forward GEMM: the input's and the weight's, the
    router's included)."""
    bt, d, L, E = cfg.bt, cfg.d, cfg.latent, cfg.n_experts
    P, I, SI = cfg.bt * cfg.top_k, cfg.expert_inter, cfg.n_shared * cfg.shared_inter
    recompute = 2 * bt * d * L + 3 * 2 * P * L * I + 2 * 2 * bt * d * SI
    grads = 2 * (2 * bt * d * L          # W_up
                 + 2 * bt * d * SI       # shared down
                 + 3 * 2 * P * L * I     # expert down, gate, up
                 + 2 * bt * d * L        # W_down_proj
                 + 2 * bt * d * E        # router
                 + 2 * 2 * bt * d * SI)  # shared gate, up
    return float(recompute + grads)


def bench_backward(args, cfg) -> int:
    """moe_backward on the workload's batch: the routing from one route() call
    (outside the timed region, as a training step takes it from its forward),
    gradients into preallocated fp32 tensors."""
    print(json.dumps(backward_line(args, cfg)), flush=True)
    return 0


def backward_line(args, cfg) -> dict:
    """The JSON line of bench_backward."""
    import torch
    torch.cuda.set_device(0)
    layer, x = device_layer(cfg, args.seed)
    gen = torch.Generator(device="cuda").manual_seed(args.seed + 7)
    dy = torch.randn((cfg.bt, cfg.d), generator=gen, device="cuda").to(torch.bfloat16)
    r = layer.route(x)
    grads = {n: torch.empty(s, dtype=torch.float32, device="cuda")
             for n, s in layer.grad_shapes(cfg.bt).items()}
    for _ in range(args.warmup):
        layer.backward(x, dy, route=r, grads=grads)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        layer.backward(x, dy, route=r, grads=grads)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1e3 / args.steps
    flops = backward_flops(cfg)
    tf = flops / (ms_step * 1e-3) / 1e12
    line = {
        "metric": "backward tokens/s (gradients of x and every weight)",
        "value": cfg.bt * args.steps / dt,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name + " backward", "bt": cfg.bt, "d": cfg.d,
                   "latent": cfg.latent, "n_experts": cfg.n_experts, "top_k": cfg.top_k,
                   "expert_inter": cfg.expert_inter, "n_shared": cfg.n_shared,
                   "shared_inter": cfg.shared_inter, "cutoff": cfg.cutoff,
                   "parallelism": "1 GPU"},
        "roofline": {"bound": "mfma", "kernel": "whole backward call", "achieved": tf,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                     "traffic": None, "flops_per_call": flops},
        "kernel_sources": kernel_source_hash(),
        # the fp64 oracle would need the experts' 30 G parameters as fp64 on the host
        "cpu_baseline": None,
    }
    del grads, layer, x, dy, r
    torch.cuda.empty_cache()
    return line


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # (100 K3 prefill steps time about 2.4 s of work: long enough for an outside
    # sampler of GPU activity to see the timed region)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="k3_prefill_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-tokens", type=int, default=128)
    ap.add_argument("--cpu-tokens-1core", type=int, default=8,
                    help="tokens of the one-core oracle timing")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the K3 decode and K3 fp8 prefill lines of the default run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--two-streams", action="store_true",
                    help="run W_down_proj and the shared experts on a second stream (the "
                         "default keeps one stream: the GEMMs fill the GPU either way, and "
                         "each kernel's time is then its own)")
    ap.add_argument("--backward", action="store_true",
                    help="time moe_backward (bf16 workloads) instead of the forward")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain 1 GiB device copy (the reference kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one MI355X: the layer runs on a single GPU, with no "
              "multi-GPU path (run with --gpus 1).", file=sys.stderr)
        return 2

    import synth
    import torch
    if args.calibrate_copy:
        torch.cuda.set_device(0)
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.config in synth.FFN_CONFIGS:
        return bench_ffn(args)

    cfg = synth.CONFIGS[args.config]
    if args.backward:
        return bench_backward(args, cfg)
    if cfg.tier_slots > 0:
        return bench_tier(args, cfg)
    torch.cuda.set_device(0)
    res = time_forward(cfg, args.seed, args.steps, args.warmup, args.two_streams,
                       want_routing=True)
    line = forward_line(cfg, args, res)
    line["routing"] = routing_stats(cfg, res)
    if not args.no_secondary and args.config == "k3_prefill_bf16":
        line["secondary"] = {}
        for name in ("k3_decode_bf16", "k3_prefill_fp8", "k3_decode_mxfp4"):
            c2 = synth.CONFIGS[name]
            r2 = time_forward(c2, args.seed, args.steps, args.warmup, False)
            l2 = forward_line(c2, args, r2)
            line["secondary"][name] = {k: l2[k] for k in ("value", "unit", "ms_per_step",
                                                           "roofline", "layer", "phases_ms")}
        # the backward of the headline workload (gradients of x and every weight)
        lb = backward_line(argparse.Namespace(seed=args.seed, steps=min(args.steps, 10),
                                              warmup=min(args.warmup, 3)), cfg)
        line["secondary"]["k3_prefill_bf16_backward"] = {
            k: lb[k] for k in ("metric", "value", "unit", "ms_per_step", "steps", "roofline")}
    del res
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.seed, args.cpu_tokens,
                                            logits=line["routing"].pop("_logits", None))
        line["cpu_baseline_1core"] = cpu_baseline(cfg, args.seed, args.cpu_tokens_1core,
                                                  threads=1)
    line["routing"].pop("_logits", None)
    print(json.dumps(line), flush=True)
    return 0


def device_layer(cfg, seed):
    """The layer's weights and tokens generated in HBM, as a StableLatentMoE."""
    import torch
    import sparse_moe_layer_quantile_amd as moe
    import synth
    lay = synth.device_layer(cfg, seed)
    layer = moe.StableLatentMoE(moe.make_config(**synth.abi_config_args(cfg)),
                                synth.abi_tensors(cfg, lay))
    torch.cuda.synchronize()
    return layer, lay["x"]


def time_forward(cfg, seed, steps, warmup, two_streams, want_routing=False):
    """steps timed forwards of the workload after warmup ones, inputs resident
    in HBM.  Wall time per step between two device synchronisations, and each
    phase's average from the HIP events the library records on the stream that
    phase runs on."""
    import torch
    import sparse_moe_layer_quantile_amd as moe
    layer, x = device_layer(cfg, seed)
    y = torch.empty((cfg.bt, cfg.d), dtype=x.dtype, device="cuda")
    side = torch.cuda.Stream() if two_streams else None
    # this batch's routing: experts touched (for the algorithmic byte count)
    _, r = layer.forward(x, shared_stream=side, return_routing=True, out=y)
    counts = r["counts"].cpu().numpy()
    extra = {}
    if want_routing:
        extra = dict(logits=r["logits"].cpu().numpy(), cutoff=r["cutoff"].cpu().numpy(),
                     idx=r["idx"].cpu().numpy())
    del r
    # warmup with phase events on, so the event pool is filled before timing
    moe.profile_enable(True)
    for _ in range(warmup):
        layer.forward(x, shared_stream=side, out=y)
    torch.cuda.synchronize()
    moe.profile_read()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.forward(x, shared_stream=side, out=y)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    phases = moe.profile_read()
    moe.profile_enable(False)
    del layer, x, y
    torch.cuda.empty_cache()
    return dict(dt=dt, steps=steps, warmup=warmup, ms_step=dt * 1e3 / steps, phases=phases,
                counts=counts, two_streams=two_streams, **extra)


def forward_line(cfg, args, res) -> dict:
    """The JSON line of one forward workload from time_forward's result."""
    import synth
    counts = res["counts"]
    touched = int((counts > 0).sum())
    phases = res["phases"]
    ms_step = res["ms_step"]
    work = phase_work(cfg, touched)
    dom = max(phases, key=lambda n: phases[n][0])
    a8 = cfg.act_quant == "mxfp8"
    # the routed experts' GEMMs on MX FP8 inputs run the block-scaled MFMA at the fp8 rate
    peak = PEAK_FP8_TFLOPS if a8 and dom.startswith("expert_") else PEAK_BF16_TFLOPS
    roof = roofline_of(dom, work[dom][0], work[dom][1], phases[dom][0], peak)
    roof["traffic"], roof["traffic_method"] = measured_traffic(cfg.name, dom)
    layer_flops = cfg.flops()
    weight_bytes = sum(sp.nbytes + (sp.n_scale_blocks * (1 if sp.dtype in synth.MX_DTYPES else 4)
                                    if sp.dtype in (synth.FP8, *synth.MX_DTYPES) else 0)
                       for n, sp in synth.specs(cfg).items() if n != "x")
    # weights a step reads: the dense ones and each touched expert once
    sp = synth.specs(cfg)
    per_expert = sum(sp[n].nbytes + (sp[n].n_scale_blocks * (1 if sp[n].dtype in synth.MX_DTYPES
                                                              else 4)
                                     if sp[n].dtype in (synth.FP8, *synth.MX_DTYPES) else 0)
                     for n in ("w_gate", "w_up", "w_down")) / cfg.n_experts
    read_bytes = weight_bytes - (cfg.n_experts - touched) * per_expert + 2 * cfg.bt * cfg.d * 2
    return {
        "metric": METRIC,
        "value": cfg.bt * res["steps"] / res["dt"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": res["steps"],
        "warmup": res["warmup"],
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (("bf16+mxfp8" if cfg.weight == "mxfp8" else "bf16+mxfp8xmxfp4") if a8
                  else "bf16") if cfg.act == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "bt": cfg.bt, "d": cfg.d, "latent": cfg.latent,
                   "n_experts": cfg.n_experts, "top_k": cfg.top_k,
                   "expert_inter": cfg.expert_inter, "n_shared": cfg.n_shared,
                   "shared_inter": cfg.shared_inter, "weights": cfg.weight,
                   "expert_inputs": "mxfp8" if a8 else cfg.act,
                   "cutoff": cfg.cutoff, "router_bias": cfg.bias,
                   "parallelism": "1 GPU", "streams": 2 if res["two_streams"] else 1},
        "roofline": roof,
        "layer": {"tflops": layer_flops / (ms_step * 1e-3) / 1e12,
                  "mfma_frac": layer_flops / (ms_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
                  "experts_touched": touched,
                  "weight_gb": weight_bytes / 1e9,
                  # weight-streaming view: every byte a step must read (touched
                  # experts once, dense weights, x and y) over the step time
                  "read_gb": read_bytes / 1e9,
                  "hbm_gbs": read_bytes / (ms_step * 1e-3) / 1e9,
                  "hbm_frac": read_bytes / (ms_step * 1e-3) / (PEAK_HBM_GBS * 1e9)},
        "phases_ms": {n: round(v[0], 4) for n, v in phases.items()},
        "kernel_sources": kernel_source_hash(),
        "cpu_baseline": None,
    }


def routing_stats(cfg, res) -> dict:
    """Per-expert load of the timed batch (max and min over the mean bt k / E)
    and its near ties: tokens whose k-th and (k+1)-th best cutoff-adjusted
    scores sigmoid(z - alpha) are within 1e-6 (the band inside which the
    selection is allowed to differ from the oracle's)."""
    counts = res["counts"].astype(np.float64)
    mean = cfg.bt * cfg.top_k / cfg.n_experts
    out = {"load_max_over_mean": float(counts.max() / mean),
           "load_min_over_mean": float(counts.min() / mean)}
    z = res.get("logits")
    if z is not None and cfg.top_k < cfg.n_experts:
        r = (z - res["cutoff"][None, :].astype(np.float32)).astype(np.float32)
        part = -np.partition(-r, (cfg.top_k - 1, cfg.top_k), axis=1)
        s = 1.0 / (1.0 + np.exp(-part[:, cfg.top_k - 1:cfg.top_k + 1].astype(np.float64)))
        out["near_tie_tokens"] = int((s[:, 0] - s[:, 1] <= 1e-6).sum())
        out["_logits"] = z
    return out


if __name__ == "__main__":
    sys.exit(main())
