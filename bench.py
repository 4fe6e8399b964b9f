#!/usr/bin/env python3
"""Benchmark of one MoE-layer forward pass on one MI355X.

A step is one moe_layer_forward (route + top-k, dispatch, expert FFN,
weighted combine) over one synthetic layer whose inputs and weights are
already resident in HBM.

The headline workload is the largest layer: the Mixtral-8x7B-shaped prefill
layer (T=8192 tokens, m=4096, p=14336, E=8, top-2, SwiGLU, bf16), whose
expert FFN is a grouped GEMM on the matrix cores.  The default run prints
one JSON line for it, with the roofline position of its dominant kernel
(timed with HIP events around its launches on the launch stream) and the CPU
oracle timed on a bounded sample of the same layer.  Beside it, under
"configs", the same figures for the other measured layers (tiny fp32,
Mixtral decode, Phi-3.5 skewed, Mixtral int8, int4, fp8, fp8a8 and MXFP4
decode, Mixtral int8, int4, fp8, fp8a8, i8a8 and MXFP4 prefill; fp8a8 and
i8a8: fp8 or int8 weights with activations quantised to the same format, the
prefill up projection on the fp8 or int8 matrix cores).

  python bench.py [--steps K] [--warmup W]            headline + every layer
  python bench.py --workload c2 [--steps K]           one layer only
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 (and int8, in TOP/s)
METRIC = "MoE layer tokens/s; achieved HBM GB/s (T≤64) or MFMA TFLOP/s (T≥4096)"
HEADLINE = "c4"
OTHERS = ["c1", "c2", "c3", "c5", "c6", "c9", "c10", "c13", "c7", "c8", "c11", "c12", "c14", "c15"]
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
_CSRC = "mixture_experts_layer_gemv_amd/csrc/"
_SKINNY = [_CSRC + f for f in
           ("moe_ffn_skinny.hip", "moe_index.hpp", "moe_dispatch_block.hpp", "moe_kernels.hpp", "moe_lds.hpp",
            "moe_convert.hpp")]
_GEMM = [_CSRC + f for f in ("moe_ffn_gemm.hip", "moe_index.hpp", "moe_kernels.hpp", "moe_lds.hpp", "moe_convert.hpp")]
_F32 = [_CSRC + f for f in ("moe_misc.hip", "moe_index.hpp", "moe_kernels.hpp")]
KERNEL_SOURCES = {"ffn_up": _SKINNY, "ffn_down": _SKINNY, "gemm_up": _GEMM, "gemm_down": _GEMM,
                  "ffn_f32_up": _F32, "ffn_f32_down": _F32}
KERNELS = ("fill", "route_topk", "dispatch", "quant_rows", "expand_w", "ffn_up", "ffn_down", "ffn_f32_up", "ffn_f32_down", "finalize",
           "pack_rows", "gemm_up", "gemm_down", "combine")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None,
                    help="time only this layer (c1..c15); default: the prefill layer with every other layer beside it")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (for PMC byte-counter calibration)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic(sp, counts):
    """Bytes and flops one forward must move/do, per kernel and for the layer.

    Only experts that received tokens count.  Weight bytes: G*m*p (gate[+up])
    and p*m (down) elements per touched expert, plus integer scales.
    Activation bytes: x read, hidden H written and read back (bf16), y
    written.  Flops: 2*m*p per row per m x p matrix (the pages' |O| rounds to
    this)."""
    wb = {"f32": 4, "bf16": 2, "i8": 1, "i8a8": 1, "i4": 0.5, "fp8": 1, "fp8a8": 1, "mxfp4": 0.5 + 1 / 32}[sp.w_dtype]
    ab = 4 if sp.x_dtype == "f32" else 2
    G = 2 if sp.kind == "swiglu" else 1
    touched = sum(1 for c in counts if c > 0)
    rows = sp.T * sp.k
    q = sp.w_dtype in ("i8", "i8a8", "i4", "fp8", "fp8a8")  # fp32 per-channel scales (MXFP4's are in wb)
    up_w = int(touched * G * sp.m * sp.p * wb) + (touched * G * sp.p * 4 if q else 0)
    dn_w = int(touched * sp.p * sp.m * wb) + (touched * sp.m * 4 if q else 0)
    h_bytes = rows * sp.p * (4 if sp.w_dtype == "f32" else 2)
    up_bytes = up_w + sp.T * sp.m * ab + h_bytes
    dn_bytes = dn_w + h_bytes + sp.T * sp.m * 4 * 2
    layer_bytes = up_w + dn_w + sp.T * sp.m * ab * 2 + sp.m * sp.E * 4
    up_flop = 2.0 * rows * G * sp.m * sp.p
    dn_flop = 2.0 * rows * sp.p * sp.m
    return dict(up_bytes=up_bytes, dn_bytes=dn_bytes, layer_bytes=layer_bytes, up_flop=up_flop, dn_flop=dn_flop,
                layer_flop=up_flop + dn_flop + 2.0 * sp.T * sp.m * sp.E, touched=touched)


def load_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel's sources changed since the counters were taken."""
    path = os.path.join(TRAFFIC_DIR, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash(kernel):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_info():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"nproc": os.cpu_count(), "affinity": affinity, "model": model}


def cpu_baseline(L, budget_s):
    """The oracle, unmodified, on whole tokens of the layer: one thread, then
    half and all of its default threads (OpenMP over tokens), each on as many
    tokens as fit its share of the budget."""
    import numpy as np

    import oracle

    sp = L["spec"]
    X = oracle.Experts.from_layer(L)
    full = oracle.max_threads()
    counts = sorted({1, max(1, full // 2), full})
    share = budget_s / len(counts)
    oracle.set_threads(1)
    t0 = time.perf_counter()
    oracle.forward_tokens(X, L["x"], L["wg"], L["bias"], sp.k, np.arange(1))
    one = max(time.perf_counter() - t0, 1e-6)
    runs = {}
    for th in counts:
        oracle.set_threads(th)
        n = int(min(sp.T, max(1, th * int(max(1.0, share / one)))))
        t0 = time.perf_counter()
        oracle.forward_tokens(X, L["x"], L["wg"], L["bias"], sp.k, np.arange(n))
        dt = time.perf_counter() - t0
        runs[th] = (n, dt, n / dt)
    oracle.set_threads(full)
    best = max(runs, key=lambda th: runs[th][2])
    n, dt, rate = runs[full]
    return {"value": round(rate, 3), "unit": "tokens/s", "cores": full, "kind": "oracle",
            "sample": f"{n} of {sp.T} tokens of the {sp.name} layer, whole forward in fp64 on {full} threads "
                      f"({dt:.2f} s)",
            "single_thread_tokens_per_s": round(runs[1][2], 4),
            "tokens_per_s_by_threads": {str(th): round(r[2], 4) for th, r in runs.items()},
            "best_threads": best, **cpu_info()}


def time_steps(fn, steps, stream=None):
    """ms per call of fn over exactly `steps` calls between two events on the
    launch stream, bracketed by device synchronisations."""
    import torch

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(steps):
        fn()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def measure(key, args, headline):
    """Generates one layer, times it, and returns its figures."""
    import torch

    import synth
    import mixture_experts_layer_gemv_amd as M
    from mixture_experts_layer_gemv_amd.layer import MoELayer

    sp = synth.spec(key)
    log(f"workload {sp.name}: generating inputs")
    L = synth.make_layer(sp)
    layer = MoELayer(L)
    dbg = layer.debug_buffers()
    y = layer.new_output()
    layer.forward(y=y, dbg=dbg)
    torch.cuda.synchronize()
    counts = dbg["counts"].cpu().tolist()
    log(f"{sp.name}: counts per expert {counts}; warmup {args.warmup}, {args.steps} timed steps")
    for _ in range(args.warmup):
        layer.forward(y=y)
    ms = time_steps(lambda: layer.forward(y=y), args.steps)

    out = {"ms_per_step": round(ms, 5), "value": round(sp.T / (ms * 1e-3), 2)}
    if headline:
        # the same K steps replayed from a HIP graph of the forward
        g, _ = layer.capture(y=y)
        for _ in range(3):
            M.moe_graph_launch(g)
        ms_graph = time_steps(lambda: M.moe_graph_launch(g), args.steps)
        M.moe_graph_destroy(g)
        # the fused forward: layer norm of x in the routing pass and a residual
        gen = torch.Generator().manual_seed(1)
        gamma = (1.0 + 0.1 * torch.randn(sp.m, generator=gen)).to("cuda")
        beta = (0.05 * torch.randn(sp.m, generator=gen)).to("cuda")
        resid = (0.5 * torch.randn(sp.T, sp.m, generator=gen)).to(y.dtype).to("cuda")
        ws = layer.ensure_workspace(sp.T)

        def fused_step():
            M.moe_layer_forward_fused(layer.handle, layer.wg, layer.bias, layer.x, layer.x_dtype, M.MOE_NORM_LAYER,
                                      gamma, beta, 1e-5, resid, sp.T, sp.m, sp.p, sp.E, sp.k, y, layer.y_dtype, ws,
                                      layer.ws_bytes)

        for _ in range(3):
            fused_step()
        ms_fused = time_steps(fused_step, args.steps)
        out["graph"] = {"ms_per_step": round(ms_graph, 5), "value": round(sp.T / (ms_graph * 1e-3), 2)}
        out["fused_norm_residual"] = {"ms_per_step": round(ms_fused, 5), "value": round(sp.T / (ms_fused * 1e-3), 2)}

    # Kernel timing: K more steps in which the library brackets every launch
    # with HIP events recorded on the stream the kernel runs on (the events
    # add small gaps between launches, so the step time is taken without them).
    M.moe_profile_begin(args.steps * 8)
    ms_events = time_steps(lambda: layer.forward(y=y), args.steps)
    M.moe_profile_end()
    kern = {}
    for name in KERNELS:
        tot, n = M.moe_profile_query(name)
        if n:
            kern[name] = round(tot / n * 1000.0, 3)  # us per launch

    A = algorithmic(sp, counts)
    dominant = next(n for n in ("gemm_up", "ffn_up", "ffn_f32_down") if n in kern)
    dom_us = kern[dominant]
    if dominant == "gemm_up":
        # fp8 activations: the up projection multiplies on the fp8 matrix
        # cores (its own peak), the down projection in bf16
        up_peak = MFMA_FP8_PEAK_TFLOPS if sp.w_dtype in ("fp8a8", "i8a8") else MFMA_BF16_PEAK_TFLOPS
        achieved = A["up_flop"] / (dom_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": up_peak,
                "unit": "TOP/s" if sp.w_dtype == "i8a8" else "TFLOP/s", "frac": round(achieved / up_peak, 4)}
        work = {"algorithmic_flop": A["up_flop"]}
        ideal_s = (A["up_flop"] / up_peak + (A["layer_flop"] - A["up_flop"]) / MFMA_BF16_PEAK_TFLOPS) / 1e12
        layer_frac = {"bound": "mfma", "tflops": round(A["layer_flop"] / (ms * 1e-3) / 1e12, 2),
                      "frac": round(ideal_s / (ms * 1e-3), 4)}
    else:
        nbytes = A["up_bytes"] if dominant == "ffn_up" else A["dn_bytes"]
        achieved = nbytes / (dom_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
        work = {"algorithmic_bytes": nbytes}
        layer_frac = {"bound": "hbm", "gbs": round(A["layer_bytes"] / (ms * 1e-3) / 1e9, 1),
                      "frac": round(A["layer_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    roof["traffic"] = load_traffic(dominant, sp.name)
    roof["kernel"] = dominant
    roof.update(work)
    roof["launch_us"] = dom_us
    out.update({
        "ms_per_step_with_kernel_events": round(ms_events, 5),
        "dtype": {"f32": "f32", "bf16": "bf16", "i8": "bf16", "i4": "bf16", "fp8": "bf16",
                  "fp8a8": "fp8" if dominant == "gemm_up" else "bf16",
                  "i8a8": "int8" if dominant == "gemm_up" else "bf16", "mxfp4": "bf16"}[sp.w_dtype],
        "config": {"workload": sp.name, "T": sp.T, "m": sp.m, "p": sp.p, "E": sp.E, "k": sp.k, "expert": sp.kind,
                   "weights": sp.w_dtype, "activations": sp.x_dtype, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "layer": {**layer_frac, "algorithmic_bytes": A["layer_bytes"], "algorithmic_flop": A["layer_flop"],
                  "touched_experts": A["touched"], "counts": counts, "kernel_us": kern},
    })
    if headline and args.copy_calib_mib:
        n = args.copy_calib_mib * (1 << 20) // 4
        # a fill (writes the buffer once), copies (read it once, write it
        # once) and sums (read it once): known byte counts for the counters
        a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        s = torch.zeros((), dtype=torch.float32, device="cuda")
        for _ in range(3):
            s += a.sum()
        torch.cuda.synchronize()
        del a, b, s
    if headline and not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(L, args.cpu_budget)
    layer.close()
    del L, layer, dbg, y
    gc.collect()
    torch.cuda.empty_cache()
    return out


def host_link_gbs(nbytes=1 << 30, reps=5):
    """Measured host -> device rate (GB/s) of a pinned buffer: beta of the
    pages' prefetch threshold."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    ev1.record()
    torch.cuda.synchronize()
    gbs = nbytes * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del src, dst
    return gbs


def measure_streamed(key, args, slots, beta_gbs):
    """The layer with its experts in host memory (moe_weights_offload, `slots`
    device slots): step time, bytes streamed per step, and the overlap of the
    copies with the expert compute, against the pages' threshold
    q* = phi * dtype / (2 beta) for hiding a transfer."""
    import torch

    import synth
    import mixture_experts_layer_gemv_amd as M
    from mixture_experts_layer_gemv_amd.layer import MoELayer

    sp = synth.spec(key)
    log(f"{sp.name}: host-resident experts, {slots} slots")
    L = synth.make_layer(sp)
    layer = MoELayer(L)
    y = layer.new_output()
    steps = max(3, min(args.steps, 10))
    for _ in range(2):
        layer.forward(y=y)
    ms_resident = time_steps(lambda: layer.forward(y=y), steps)
    layer.offload(slots)
    for _ in range(2):
        layer.forward(y=y)
    h0, m0, b0 = M.moe_weights_offload_stats(layer.handle)
    ms = time_steps(lambda: layer.forward(y=y), steps)
    h1, m1, b1 = M.moe_weights_offload_stats(layer.handle)
    layer.close()
    del L, layer, y
    gc.collect()
    torch.cuda.empty_cache()
    bytes_step = (b1 - b0) / steps
    transfer_ms = bytes_step / (beta_gbs * 1e9) * 1e3
    wb = {"bf16": 2, "i8": 1, "i8a8": 1, "i4": 0.5, "fp8": 1, "fp8a8": 1, "mxfp4": 0.5}[sp.w_dtype]
    q_star = MFMA_BF16_PEAK_TFLOPS * 1e12 * wb / (2 * beta_gbs * 1e9)
    hidden = (transfer_ms + ms_resident - ms) / max(min(transfer_ms, ms_resident), 1e-9)
    return {"workload": sp.name, "slots": slots, "ms_per_step": round(ms, 3), "value": round(sp.T / (ms * 1e-3), 2),
            "resident_ms_per_step": round(ms_resident, 4), "h2d_bytes_per_step": int(bytes_step),
            "expert_misses_per_step": round((m1 - m0) / steps, 2), "expert_hits_per_step": round((h1 - h0) / steps, 2),
            "host_link_gbs": round(beta_gbs, 2), "transfer_ms_per_step": round(transfer_ms, 3),
            "overlap_of_shorter": round(max(0.0, min(1.0, hidden)), 3),
            "rows_per_expert": round(sp.T * sp.k / sp.E, 1), "q_star_rows": round(q_star)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py: the layer runs on one GPU; --gpus {max(args.gpus, world)} is not "
              "supported (multi-GPU sharding is a design note only).", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_layer_gemv_amd as M

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    M.lib()
    head_key = args.workload or HEADLINE
    head = measure(head_key, args, headline=True)
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "data": "synthetic",
    }
    out.update({k: v for k, v in head.items() if k not in out})
    if args.workload is None:
        out["configs"] = {}
        for key in OTHERS:
            r = measure(key, args, headline=False)
            out["configs"][r["config"]["workload"]] = {
                k: r[k] for k in ("ms_per_step", "value", "dtype", "config", "roofline", "layer")}
        beta = host_link_gbs()
        out["host_streamed"] = [measure_streamed(key, args, 4, beta) for key in ("c2", "c4")]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
