#!/usr/bin/env python3
"""Throughput of the DeepSeekMoE layer forward on one MI355X.

One step = one moe_layer_forward (router, dispatch, gate/up GEMM, down GEMM,
shared expert, combine) over one batch of seeded synthetic inputs already
resident in HBM. Default workload: the DeepSeek-V3-shaped prefill layer
(T=16384, D=7168, 256 routed experts of hidden 2048 in 8 groups keep 4,
top-8 sigmoid routing with selection bias, 1 shared expert), bf16.
Reported: routed tokens/s, % of bf16 MFMA peak, the dominant kernel's
roofline, the fp8 decode-shaped layer's HBM GB/s, and the CPU oracle's rate
on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed tokens/s per MoE layer (V3-shape T=16384) + %MFMA peak; decode HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# HBM traffic of one gate/up GEMM launch on the V3 prefill workload, from two
# rocprofv3 --pmc runs of this bench (FETCH_SIZE, then WRITE_SIZE; KiB per
# dispatch, mean of the dispatches after the first, cold one), each scaled by
# what the same counter reads for the bench's 1 GiB device-to-device copy probe
# (FETCH_SIZE 524317.1 KiB for 1048576 KiB read; WRITE_SIZE 1048576 KiB for
# 1048576 KiB written).
# Valid only for the kernel sources with these hashes; otherwise reported null.
GATEUP_COUNTERS = {
    "sources": {"mixture_experts_layer_38_amd/csrc/grouped_gemm.hip":
                "53380366932379c1cfb8fb77270e07d4365b3e3562d5e59ee849be5b42cb3642",
                "mixture_experts_layer_38_amd/csrc/moe_internal.hpp":
                "d8bec0ef68504479c6f90c9ed087ca29354afba77a4f08124880edeb162eec8d"},
    "workload": "v3_prefill",
    "fetch_kib": 15954495.3, "write_kib": 589824.0,
    "fetch_scale": 1048576.0 / 524317.1, "write_scale": 1.0,
}


# the same two counters for the fp8 decode layer's gate/up streaming kernel
# (stream_gemm_kernel<true, 0>, decode workload run in the prefill slot:
# `bench.py --config v3_decode_fp8`; the same 1 GiB copy calibrates FETCH_SIZE)
DECODE_GATEUP_COUNTERS = {
    "sources": {"mixture_experts_layer_38_amd/csrc/stream_gemm.hip":
                "d646320d0c203bdc1648a7b193650f720e6f99e7c13b942fcfaf152206d49473",
                "mixture_experts_layer_38_amd/csrc/moe_internal.hpp":
                "d8bec0ef68504479c6f90c9ed087ca29354afba77a4f08124880edeb162eec8d"},
    "workload": "v3_decode_fp8",
    "fetch_kib": 1829744.4, "write_kib": 2562.7,
    "fetch_scale": 1048576.0 / 524314.8, "write_scale": 1.0,
}


def pinned_traffic(c, cfg):
    """Calibrated HBM bytes per launch from counter figures c, or None when they
    do not describe the kernel that was built (or another workload)."""
    import hashlib
    if cfg.name != c["workload"]:
        return None
    for rel, digest in c["sources"].items():
        with open(os.path.join(ROOT, rel), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != digest:
                return None
    return round((c["fetch_kib"] * c["fetch_scale"] + c["write_kib"] * c["write_scale"]) * 1024)


def gateup_traffic(cfg):
    """Calibrated HBM bytes per gate/up GEMM launch (prefill), or None."""
    return pinned_traffic(GATEUP_COUNTERS, cfg)


def gateup_algorithmic_bytes(cfg):
    """Each operand byte once: routed and shared gate/up weights, the gathered
    token rows (T*K routed + T shared), and h written; e4m3 operands count one
    byte per element plus their fp32 block scales."""
    wb = 1 if cfg.weight == "fp8" else 2
    ab = 1 if cfg.act_quant else 2
    wrows = cfg.E * 2 * cfg.H + 2 * cfg.Hs
    w = wb * wrows * cfg.D + (4 * (wrows // 128) * (cfg.D // 128) if cfg.weight == "fp8" else 0)
    xrows = cfg.T * cfg.K + cfg.T
    x = ab * xrows * cfg.D + (4 * xrows * (cfg.D // 128) if cfg.act_quant else 0)
    hel = cfg.T * cfg.K * cfg.H + cfg.T * cfg.Hs
    h = ab * hel + (4 * hel // 128 if cfg.act_quant else 0)
    return w + x + h


def mfma_flops(cfg, T=None):
    T = cfg.T if T is None else T
    return 2.0 * T * (cfg.K * 3 * cfg.D * cfg.H + 3 * cfg.D * cfg.Hs)


def gateup_flops(cfg):
    return 2.0 * cfg.T * (cfg.K * 2 * cfg.D * cfg.H + 2 * cfg.D * cfg.Hs)


def backward_flops(cfg):
    """MFMA work of the backward pass: the gate/up recompute, the two data
    gradients and the two weight gradients of the experts (each as much as
    the forward's product), and the router's two products (E padded to 64)."""
    ep = (cfg.E + 63) // 64 * 64
    return gateup_flops(cfg) + 2 * mfma_flops(cfg) + 4.0 * cfg.T * ep * cfg.D


def run_backward(args, torch, M, cfg, inp):
    """Backward steps on the forward's inputs: fp32 gradients of every expert,
    the shared expert, gate_w and x for a random d_out (HIP events on the
    stream the library runs on)."""
    layer = M.MoELayer.from_config(cfg, backward=True)
    d_out = torch.randn((cfg.T, cfg.D), generator=torch.Generator(device="cuda").manual_seed(8), device="cuda")
    for _ in range(2):
        g = layer.backward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared, d_out)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(3, args.steps // 4)
    ev0.record()
    for _ in range(n):
        g = layer.backward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared, d_out)
    ev1.record()
    ev1.synchronize()
    ms = ev0.elapsed_time(ev1) / n
    flop = backward_flops(cfg)
    log(f"backward: {ms:.3f} ms/step ({n} steps)")
    # a training step whose forward keeps the gate/up products ([a | u] and
    # g * h, from the same accumulators as h): the training forward, then the
    # backward that reads them instead of recomputing them
    out = torch.empty((cfg.T, cfg.D), dtype=torch.float32, device="cuda")
    args_f = (inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared)

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / n

    def train_step():
        layer.forward(*args_f, out=out, train=True)
        return layer.backward(*args_f, d_out, saved=True)

    for _ in range(2):
        g = train_step()
    torch.cuda.synchronize()
    step_ms = timed(train_step)
    fwd_ms = timed(lambda: layer.forward(*args_f, out=out, train=True))
    bwd_ms = timed(lambda: layer.backward(*args_f, d_out, saved=True))
    flop_saved = flop - gateup_flops(cfg)
    saved_bytes = 2 * (cfg.T * cfg.K * 3 * cfg.H + cfg.T * 3 * cfg.Hs)
    log(f"training step with saved gate/up products: {step_ms:.3f} ms (forward {fwd_ms:.3f}, backward {bwd_ms:.3f})")
    del g, layer, out
    torch.cuda.empty_cache()
    return {"ms": round(ms, 4), "steps": n, "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
            "mfma_flop": flop, "achieved_tflops": round(flop / (ms * 1e-3) / 1e12, 2),
            "frac_of_bf16_peak": round(flop / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4),
            "gradients": "fp32 (x, gate_w, every expert, shared expert)",
            "recompute": "the gate/up products ([a | u], g * h) recomputed inside the backward",
            "saved_products": {
                "train_step_ms": round(step_ms, 4), "forward_train_ms": round(fwd_ms, 4),
                "backward_ms": round(bwd_ms, 4), "backward_mfma_flop": flop_saved,
                "backward_frac_of_bf16_peak": round(flop_saved / (bwd_ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4),
                "saved_bytes": saved_bytes,
                "what": "forward keeps [a | u] and g * h (bf16); backward reads them instead of recomputing"}}


def gen_progress(cfg, torch):
    """Logs every 32 experts, so that a slow generation (under a counter
    profiler every dispatch is serialised) still shows its progress."""
    def cb(e):
        if (e + 1) % 32 == 0 or e + 1 == cfg.E:
            torch.cuda.synchronize()
            log(f"  experts {e + 1}/{cfg.E} generated")
    return cb


def run_prefill(args, torch, M, MI):
    cfg = MI.CONFIGS[args.config]
    log(f"generating {cfg.name} inputs on the GPU")
    inp = MI.make_layer(cfg, "cuda", progress=gen_progress(cfg, torch))
    layer = M.MoELayer.from_config(cfg)
    out = torch.empty((cfg.T, cfg.D), dtype=torch.float32, device="cuda")
    counts = torch.empty((cfg.E,), dtype=torch.int32, device="cuda")

    def step():
        layer.forward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared, out=out, expert_counts=counts)

    for i in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")
    # the timed steps run without per-stage events (each event between two
    # stages leaves a gap of about 5 us between their kernels) ...
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    # ... and an equal pass with them gives the per-stage split
    layer.set_stage_timing(True)
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    stages, calls = layer.stage_times()
    layer.set_stage_timing(False)
    stage_avg = {k: v / max(calls, 1) for k, v in stages.items()}
    log(f"{args.steps} steps: {ms:.3f} ms/step; stages {stage_avg}")
    # load balance between steps on this step's counts (bias update + statistics)
    bias = (inp.sel_bias.clone() if inp.sel_bias is not None
            else torch.zeros(cfg.E, dtype=torch.float32, device="cuda"))
    for _ in range(10):
        M.bias_update(counts, bias, 1e-3)
        M.load_stats(counts)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(200):
        M.bias_update(counts, bias, 1e-3)
        M.load_stats(counts)
    ev1.record()
    ev1.synchronize()
    balance_us = ev0.elapsed_time(ev1) * 1e3 / 200
    g1_ms = stage_avg["gate_up_gemm"]
    g1_tflops = gateup_flops(cfg) / (g1_ms * 1e-3) / 1e12
    # e4m3 activations multiply on the fp8 matrix cores (their own peak); the
    # gate/up stage then also holds the token-row quantiser
    peak = PEAK_FP8_TFLOPS if cfg.act_quant else PEAK_BF16_TFLOPS
    kernel = ("grouped_gemm_f8_kernel<0> (gate/up + SwiGLU + h to e4m3; stage includes quant_e4m3_kernel)"
              if cfg.act_quant else "grouped_gemm_bf16_kernel<0> (gate/up + SwiGLU)")
    res = dict(cfg=cfg, inp=inp, ms=ms, stages=stage_avg, counts=counts.cpu().tolist(), balance_us=balance_us,
               mfma_frac=mfma_flops(cfg) / (ms * 1e-3) / (peak * 1e12),
               roofline=dict(bound="mfma", achieved=round(g1_tflops, 2), peak=peak, unit="TFLOP/s",
                             frac=round(g1_tflops / peak, 4), traffic=gateup_traffic(cfg),
                             traffic_unit="HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                             algorithmic_bytes=gateup_algorithmic_bytes(cfg),
                             kernel=kernel, per_launch_flop=gateup_flops(cfg), avg_ms=round(g1_ms, 4)))
    del layer, out
    torch.cuda.empty_cache()
    if not args.no_backward and cfg.weight == "bf16" and cfg.act == "bf16" and not cfg.act_quant:
        res["backward"] = run_backward(args, torch, M, cfg, inp)
    return res


def run_config(args, torch, M, MI, name):
    """One of the other workloads: W warm-ups, then K steps timed end to end
    (HIP events on the library's stream, no per-stage events), then an equal
    pass with per-stage events for the gate/up kernel's roofline."""
    cfg = MI.CONFIGS[name]
    inp = MI.make_layer(cfg, "cuda")
    layer = M.MoELayer.from_config(cfg)
    out = torch.empty((cfg.T, cfg.D), dtype=torch.float32, device="cuda")
    counts = torch.empty((cfg.E,), dtype=torch.int32, device="cuda")

    def step():
        layer.forward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared, out=out, expert_counts=counts)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        step()
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b) / args.steps
    layer.set_stage_timing(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    stages, calls = layer.stage_times()
    layer.set_stage_timing(False)
    stage_avg = {k: v / max(calls, 1) for k, v in stages.items()}
    flop = mfma_flops(cfg)
    res = dict(T=cfg.T, ms_per_step=round(ms, 4), routed_tokens_per_s=round(cfg.T / (ms * 1e-3), 1),
               assignments_per_s=round(cfg.T * cfg.K / (ms * 1e-3), 1),
               stages_ms={k: round(v, 4) for k, v in stage_avg.items()})
    if cfg.weight == "f32":
        # the tiny fp32 layer: seven launches of a few microseconds each
        res["bound"] = "launch latency"
        res["expert_flop"] = flop
    else:
        g1 = stage_avg["gate_up_gemm"]
        res["mfma_frac"] = round(flop / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4)
        res["roofline"] = dict(bound="mfma", kernel="grouped_gemm_bf16_kernel<0> (gate/up + SwiGLU)",
                               achieved=round(gateup_flops(cfg) / (g1 * 1e-3) / 1e12, 2), peak=PEAK_BF16_TFLOPS,
                               unit="TFLOP/s", frac=round(gateup_flops(cfg) / (g1 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                               per_launch_flop=gateup_flops(cfg), avg_ms=round(g1, 4))
    log(f"{name}: {ms:.4f} ms/step, stages {res['stages_ms']}")
    del layer, inp, out
    torch.cuda.empty_cache()
    return res


def decode_bytes(cfg, n_touched):
    E, D, H, Hs = cfg.E, cfg.D, cfg.H, cfg.Hs
    per_expert = 3 * H * D + 4 * ((2 * H // 128) * (D // 128) + (D // 128) * (H // 128))
    shared = 3 * Hs * D + 4 * ((2 * Hs // 128) * (D // 128) + (D // 128) * (Hs // 128))
    gate_up = n_touched * (2 * H * D + 4 * (2 * H // 128) * (D // 128)) + 2 * Hs * D + 4 * (2 * Hs // 128) * (D // 128)
    total = n_touched * per_expert + shared + E * D * 4 + E * 4 + cfg.T * D * 2 + cfg.T * D * 4
    return total, gate_up


def run_decode(args, torch, M, MI):
    cfg = MI.CONFIGS[args.decode_config]
    log(f"generating {cfg.name} inputs on the GPU")
    inp = MI.make_layer(cfg, "cuda", progress=gen_progress(cfg, torch))
    layer = M.MoELayer.from_config(cfg)
    out = torch.empty((cfg.T, cfg.D), dtype=torch.float32, device="cuda")
    counts = torch.empty((cfg.E,), dtype=torch.int32, device="cuda")
    # Between steps a 1 GiB read (> the 256 MiB memory-side cache) evicts the
    # weights; a read leaves no dirty lines, whose write-back would otherwise
    # fall inside the next timed step. The median after a 1 GiB write is
    # reported beside it.
    evict = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    def clean_evict(i):
        torch.sum(evict, dim=0, out=sink)

    def dirty_evict(i):
        evict.fill_(float(i))

    def step():
        layer.forward(inp.x, inp.gate_w, inp.sel_bias, inp.experts, inp.shared, out=out, expert_counts=counts)

    for i in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # step time without the per-stage events (recording them between the
    # stages costs about 20 us of a 1.1 ms decode step) ...
    def timed(ev):
        times = []
        for i in range(args.steps):
            ev(i)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            step()
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b))
        return times

    times_dirty = timed(dirty_evict)
    evict.fill_(1.0)
    times = timed(clean_evict)
    # ... and the per-stage split from an equal pass with them
    layer.set_stage_timing(True)
    for i in range(args.steps):
        clean_evict(i)
        step()
    torch.cuda.synchronize()
    stages, calls = layer.stage_times()
    layer.set_stage_timing(False)
    stage_avg = {k: v / max(calls, 1) for k, v in stages.items()}
    n_touched = int((counts > 0).sum())
    total, gu = decode_bytes(cfg, n_touched)
    ms = sorted(times)[len(times) // 2]
    log(f"decode: median {ms:.4f} ms, touched {n_touched}, stages {stage_avg}")
    g1 = stage_avg["gate_up_gemm"]
    del layer, inp, evict
    torch.cuda.empty_cache()
    ms_dirty = sorted(times_dirty)[len(times_dirty) // 2]
    return dict(workload=cfg.name, T=cfg.T, ms_median=round(ms, 4), ms_min=round(min(times), 4),
                ms_median_after_write_flush=round(ms_dirty, 4),
                eviction="1 GiB read before each step (a 1 GiB write instead: ms_median_after_write_flush)",
                experts_touched=n_touched, algorithmic_bytes=total, hbm_gbs=round(total / (ms * 1e-3) / 1e9, 1),
                hbm_frac=round(total / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                stages_ms={k: round(v, 4) for k, v in stage_avg.items()},
                roofline=dict(bound="hbm", kernel="stream_gemm_kernel<fp8, gate/up + SwiGLU>",
                              achieved=round(gu / (g1 * 1e-3) / 1e9, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                              frac=round(gu / (g1 * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), per_launch_bytes=gu,
                              traffic=pinned_traffic(DECODE_GATEUP_COUNTERS, cfg),
                              traffic_unit="HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                              avg_ms=round(g1, 4)))


def cpu_baseline(res, n_experts):
    """The CPU oracle, as it stands, on a bounded sample of the same workload,
    timed in two stages with every weight decoded before the clock starts:
    routing (O.route) over all T tokens, and the expert FFN (O.swiglu_ffn,
    the oracle's per-expert evaluation) for every token routed to each of
    n_experts seeded experts (all experts the routing used when n_experts is
    None) plus the shared expert on as many tokens. Experts are decoded one at
    a time, so host memory holds one expert's float64 weights. The stage times
    per token are then combined into routed tokens/s: a token needs its
    routing, K routed expert FFNs and the shared FFN."""
    import numpy as np

    from oracle import adapter as A
    from oracle import moe_oracle as O
    cfg, inp = res["cfg"], res["inp"]
    u = A.decode_tensor(inp.x)
    gw = A.decode_tensor(inp.gate_w)
    bias = None if inp.sel_bias is None else A.decode_tensor(inp.sel_bias)
    p = A.router_params(cfg)
    t0 = time.perf_counter()
    R = O.route(u, gw, bias, p)
    t_route = time.perf_counter() - t0
    idx = R["idx"]
    used = np.nonzero(np.bincount(idx.ravel(), minlength=cfg.E))[0]
    if n_experts is None or n_experts >= len(used):
        experts = used
    else:
        experts = np.sort(np.random.default_rng(0).choice(used, size=n_experts, replace=False))
    fn = A.routed_expert_fn(inp.experts)
    t_routed, pairs = 0.0, 0
    for e in experts:
        w = fn(int(e))  # decoded before the clock
        rows = u[np.nonzero((idx == e).any(axis=1))[0]]
        t0 = time.perf_counter()
        O.swiglu_ffn(rows, *w)
        t_routed += time.perf_counter() - t0
        pairs += len(rows)
        del w
    t_shared, n_sh = 0.0, 0
    if inp.shared is not None:
        sw = A.shared_expert_fn(inp.shared)()
        n_sh = min(cfg.T, max(1, pairs // cfg.K))
        t0 = time.perf_counter()
        O.swiglu_ffn(u[:n_sh], *sw)
        t_shared = time.perf_counter() - t0
    per_tok_route = t_route / cfg.T
    per_tok_ffn = cfg.K * t_routed / pairs + (t_shared / n_sh if n_sh else 0.0)
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    return dict(value=round(1.0 / (per_tok_route + per_tok_ffn), 4), unit="routed tokens/s", cores=int(cores),
                kind="oracle",
                sample=(f"{cfg.name}: routing of all {cfg.T} tokens ({t_route:.1f} s); routed FFNs of the "
                        f"{pairs} (token, expert) pairs of {len(experts)} experts ({t_routed:.1f} s) and "
                        f"the shared FFN of {n_sh} tokens ({t_shared:.1f} s), float64, weights decoded before "
                        f"the clock; value = 1 / (routing + K routed FFNs + shared FFN) per token"),
                routing_tokens_per_s=round(1.0 / per_tok_route, 1),
                ffn_tokens_per_s=round(1.0 / per_tok_ffn, 4),
                seconds=round(t_route + t_routed + t_shared, 2))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="v3_prefill")
    ap.add_argument("--decode-config", default="v3_decode_fp8")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the backward pass")
    ap.add_argument("--cpu-experts", type=int, default=None,
                    help="experts whose routed FFNs the CPU baseline times (default: every expert "
                         "the routing used, about 10 s of float64 work on 16 host threads at V3 size)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the tiny, group-limited and V2-shaped workloads")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one plain 1 GiB device-to-device copy first (a known-size reference "
                         "for hardware byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this layer forward is built and timed on a single MI355X "
              "(--gpus 1). Expert-parallel sharding over several GPUs is a design, not a built path.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_layer_38_amd as M
    import moe_inputs as MI
    M.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("copy probe: 1 GiB read + 1 GiB written")
    res = run_prefill(args, torch, M, MI)
    cfg = res["cfg"]
    line = {
        "metric": METRIC,
        "value": round(cfg.T / (res["ms"] * 1e-3), 1),
        "unit": "routed tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if cfg.act_quant else "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "D": cfg.D, "E": cfg.E, "H": cfg.H, "G": cfg.G,
                   "topk_group": cfg.kg, "K": cfg.K, "Hs": cfg.Hs, "score": cfg.score_fn,
                   "weights": cfg.weight, "activations": "e4m3 1x128" if cfg.act_quant else cfg.act,
                   "parallelism": "single GPU"},
        "mfma_frac": round(res["mfma_frac"], 4),
        "stages_ms": {k: round(v, 4) for k, v in res["stages"].items()},
        "balance_update_and_stats_us": round(res["balance_us"], 2),
        "roofline": res["roofline"],
    }
    if "backward" in res:
        line["backward"] = res["backward"]
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle (routing of every token, FFNs of {args.cpu_experts or 'all'} experts)")
        line["cpu_baseline"] = cpu_baseline(res, args.cpu_experts)
        log(f"cpu baseline: {line['cpu_baseline']}")
    del res
    torch.cuda.empty_cache()
    if not args.no_decode:
        line["decode"] = run_decode(args, torch, M, MI)
    if not args.no_other_configs:
        line["configs"] = {n: run_config(args, torch, M, MI, n) for n in ("tiny_f32", "group_bf16", "v2_prefill")}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
