#!/usr/bin/env python3
"""Benchmark of one MoE-layer forward pass on one MI355X.

A step is one moe_layer_forward (route + top-k, dispatch, expert FFN,
weighted combine) over one synthetic layer whose inputs and weights are
already resident in HBM.  Default workload: the Mixtral-8x7B-shaped decode
layer (T=16 tokens, m=4096, p=14336, E=8, top-2, SwiGLU, bf16).  Prints one
JSON line: throughput (tokens/s), the roofline position of the dominant
kernel (timed with HIP events around its launches inside the timed region),
and the CPU oracle timed on a bounded sample of the same layer.

  python bench.py [--steps K] [--warmup W] [--workload c2|c1|c3|c4|c5|c6]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
METRIC = "MoE layer tokens/s; achieved HBM GB/s (T≤64) or MFMA TFLOP/s (T≥4096)"
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
_SKINNY = ["mixture_experts_layer_gemv_amd/csrc/" + f for f in
           ("moe_ffn_skinny.hip", "moe_index.hpp", "moe_dispatch_block.hpp", "moe_kernels.hpp", "moe_lds.hpp")]
_GEMM = ["mixture_experts_layer_gemv_amd/csrc/" + f for f in
         ("moe_ffn_gemm.hip", "moe_index.hpp", "moe_kernels.hpp", "moe_lds.hpp")]
KERNEL_SOURCES = {"ffn_up": _SKINNY, "ffn_down": _SKINNY, "gemm_up": _GEMM, "gemm_down": _GEMM}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2", help="c1..c5, or c6 (int4 decode, a next row) (default c2: Mixtral decode, T=16)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (for PMC byte-counter calibration)")
    return ap.parse_args()


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic(sp, counts):
    """Bytes and flops one forward must move/do, per kernel and for the layer.

    Only experts that received tokens count.  Weight bytes: G*m*p (gate[+up])
    and p*m (down) elements per touched expert, plus int8 scales.  Activation
    bytes: x read, hidden H written and read back (bf16), y written.
    Flops: 2*m*p per row per m x p matrix (the pages' |O| rounds to this)."""
    wb = {"f32": 4, "bf16": 2, "i8": 1, "i4": 0.5}[sp.w_dtype]
    ab = 4 if sp.x_dtype == "f32" else 2
    G = 2 if sp.kind == "swiglu" else 1
    touched = sum(1 for c in counts if c > 0)
    rows = sp.T * sp.k
    q = sp.w_dtype in ("i8", "i4")
    up_w = int(touched * G * sp.m * sp.p * wb) + (touched * G * sp.p * 4 if q else 0)
    dn_w = int(touched * sp.p * sp.m * wb) + (touched * sp.m * 4 if q else 0)
    h_bytes = rows * sp.p * (4 if sp.w_dtype == "f32" else 2)
    up_bytes = up_w + sp.T * sp.m * ab + h_bytes
    dn_bytes = dn_w + h_bytes + sp.T * sp.m * 4 * 2  # fp32 accumulator read-modify-write
    layer_bytes = up_w + dn_w + sp.T * sp.m * ab * 2 + sp.m * sp.E * 4
    up_flop = 2.0 * rows * G * sp.m * sp.p
    dn_flop = 2.0 * rows * sp.p * sp.m
    return dict(up_bytes=up_bytes, dn_bytes=dn_bytes, layer_bytes=layer_bytes, up_flop=up_flop, dn_flop=dn_flop,
                layer_flop=up_flop + dn_flop + 2.0 * sp.T * sp.m * sp.E, touched=touched)


def load_traffic(kernel, workload):
    path = os.path.join(TRAFFIC_DIR, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash(kernel):
        return None  # the kernel changed since the counters were taken
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(L, budget_s):
    """The oracle, unmodified, on as many whole tokens of the layer as fit the budget."""
    import numpy as np

    import oracle

    sp = L["spec"]
    X = oracle.Experts.from_layer(L)
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.forward_tokens(X, L["x"], L["wg"], L["bias"], sp.k, np.arange(1))
    one = time.perf_counter() - t0
    # tokens run in parallel, one per thread
    n = int(max(1, min(sp.T, threads * max(1, int(budget_s / max(one, 1e-6))))))
    n = min(n, sp.T)
    toks = np.arange(n)
    t0 = time.perf_counter()
    oracle.forward_tokens(X, L["x"], L["wg"], L["bias"], sp.k, toks)
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": int(min(threads, n)), "kind": "oracle",
            "sample": f"{n} of {sp.T} tokens of the {sp.name} layer, whole forward in fp64 ({dt:.2f} s)"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py: the layer runs on one GPU; --gpus {max(args.gpus, world)} is not "
              "supported (multi-GPU sharding is a design note only).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import mixture_experts_layer_gemv_amd as M
    from mixture_experts_layer_gemv_amd.layer import MoELayer

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    M.lib()
    sp = synth.spec(args.workload)
    print(f"[bench] workload {sp.name}: generating inputs", file=sys.stderr, flush=True)
    L = synth.make_layer(sp)
    layer = MoELayer(L)
    dbg = layer.debug_buffers()
    y = layer.new_output()
    layer.forward(y=y, dbg=dbg)
    torch.cuda.synchronize()
    counts = dbg["counts"].cpu().tolist()
    print(f"[bench] counts per expert: {counts}; warmup {args.warmup}", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        layer.forward(y=y)
    torch.cuda.synchronize()

    # Timed region: exactly K steps between two events on the launch stream,
    # bracketed by device synchronisations.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        layer.forward(y=y)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps

    # The same K steps replayed from a HIP graph of the forward
    # (moe_layer_graph_create: the launches recorded once, one graph launch
    # per step), on the same stream between the same kind of events.
    g, _ = layer.capture(y=y)
    for _ in range(3):
        M.moe_graph_launch(g)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        M.moe_graph_launch(g)
    ev1.record()
    torch.cuda.synchronize()
    ms_graph = ev0.elapsed_time(ev1) / args.steps
    M.moe_graph_destroy(g)

    # The fused forward (moe_layer_forward_fused): layer norm of x in the
    # routing pass and a residual added at the end, K steps.
    gen = torch.Generator().manual_seed(1)
    gamma = (1.0 + 0.1 * torch.randn(sp.m, generator=gen)).to("cuda")
    beta = (0.05 * torch.randn(sp.m, generator=gen)).to("cuda")
    resid = (0.5 * torch.randn(sp.T, sp.m, generator=gen)).to(y.dtype).to("cuda")
    ws = layer.ensure_workspace(sp.T)

    def fused_step():
        M.moe_layer_forward_fused(layer.handle, layer.wg, layer.bias, layer.x, layer.x_dtype, M.MOE_NORM_LAYER, gamma,
                                  beta, 1e-5, resid, sp.T, sp.m, sp.p, sp.E, sp.k, y, layer.y_dtype, ws,
                                  layer.ws_bytes)

    for _ in range(3):
        fused_step()
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        fused_step()
    ev1.record()
    torch.cuda.synchronize()
    ms_fused = ev0.elapsed_time(ev1) / args.steps

    # Kernel timing: K more steps in which the library brackets every launch
    # with HIP events recorded on the stream the kernel runs on.  (The events
    # add small gaps between launches, so the step time above is taken
    # without them.)
    M.moe_profile_begin(args.steps * 8)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        layer.forward(y=y)
    ev1.record()
    torch.cuda.synchronize()
    M.moe_profile_end()
    ms_events = ev0.elapsed_time(ev1) / args.steps
    kern = {}
    for name in ("fill", "route_topk", "dispatch", "ffn_up", "ffn_down", "ffn_f32_up", "ffn_f32_down", "finalize",
                 "pack_rows", "gemm_up", "gemm_down", "combine"):
        tot, n = M.moe_profile_query(name)
        if n:
            kern[name] = round(tot / n * 1000.0, 3)  # us per launch

    if args.copy_calib_mib:
        n = args.copy_calib_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    A = algorithmic(sp, counts)
    dominant = next(n for n in ("gemm_up", "ffn_up", "ffn_f32_up") if n in kern)
    up_us = kern.get(dominant, float("nan"))
    mfma_bound = dominant == "gemm_up"
    if mfma_bound:
        achieved = A["up_flop"] / (up_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        achieved = A["up_bytes"] / (up_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["traffic"] = load_traffic(dominant, sp.name)
    roof["kernel"] = dominant
    roof["algorithmic_bytes" if not mfma_bound else "algorithmic_flop"] = (
        A["up_bytes"] if not mfma_bound else A["up_flop"])
    roof["launch_us"] = up_us

    out = {
        "metric": METRIC,
        "value": round(sp.T / (ms * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "ms_per_step_with_kernel_events": round(ms_events, 5),
        "graph": {"ms_per_step": round(ms_graph, 5), "value": round(sp.T / (ms_graph * 1e-3), 2)},
        "fused_norm_residual": {"ms_per_step": round(ms_fused, 5), "value": round(sp.T / (ms_fused * 1e-3), 2)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "i8": "bf16", "i4": "bf16"}[sp.w_dtype],
        "data": "synthetic",
        "config": {"workload": sp.name, "T": sp.T, "m": sp.m, "p": sp.p, "E": sp.E, "k": sp.k, "expert": sp.kind,
                   "weights": sp.w_dtype, "activations": sp.x_dtype, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "layer": {"hbm_gbs": round(A["layer_bytes"] / (ms * 1e-3) / 1e9, 1),
                  "tflops": round(A["layer_flop"] / (ms * 1e-3) / 1e12, 3),
                  "algorithmic_bytes": A["layer_bytes"], "touched_experts": A["touched"],
                  "counts": counts, "kernel_us": kern},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(L, args.cpu_budget)
    layer.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
