"""Shared helpers for the GPU parity tests (HIP path vs the CPU oracle)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth
from mixture_experts_layer_gemv_amd.layer import MoELayer, to_device

# Parity bars.  bf16 weights/activations with fp32 accumulation:
#   max|gpu - oracle| <= 2e-2 * max|oracle| + 1e-3
# fp32 layers: max|gpu - oracle| <= 1e-4 * max|oracle| (normwise).
BF16_REL, BF16_ABS = 2e-2, 1e-3
F32_REL = 1e-4
# Gate weights: fp32 expf/division against the oracle's double, stored fp32.
W_ABS = 2e-6


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def spec(T, m, p, E, k, kind="swiglu", w_dtype="bf16", seed=0, zipf=None, sw=0.02, sr=0.02):
    x_dtype = "f32" if w_dtype == "f32" else "bf16"
    return synth.LayerSpec("case", T, m, p, E, k, kind, x_dtype, w_dtype, seed, sigma_router=sr, sigma_w=sw,
                           zipf_s=zipf)


def bound(y_gpu, y_ref, w_dtype):
    """Returns (max error, allowed)."""
    y_ref = np.asarray(y_ref, np.float64)
    err = float(np.max(np.abs(np.asarray(y_gpu, np.float64) - y_ref))) if y_ref.size else 0.0
    scale = float(np.max(np.abs(y_ref))) if y_ref.size else 0.0
    allowed = F32_REL * scale if w_dtype == "f32" else BF16_REL * scale + BF16_ABS
    return err, allowed


def assert_close(y_gpu, y_ref, w_dtype, what=""):
    err, allowed = bound(y_gpu, y_ref, w_dtype)
    rel_rms = float(np.sqrt(np.mean((np.asarray(y_gpu, np.float64) - y_ref) ** 2)) /
                    max(np.sqrt(np.mean(np.asarray(y_ref, np.float64) ** 2)), 1e-300)) if np.size(y_ref) else 0.0
    log(f"  {what}: max|err|={err:.3e} allowed={allowed:.3e} rel_rms={rel_rms:.3e}")
    assert err <= allowed, f"{what}: max error {err} > {allowed}"
    return err


def logit_bound(x64, wg, bias):
    """fp32 worst-case bound for a length-m dot product plus bias, plus one rounding of the oracle."""
    m = x64.shape[1]
    mag = np.abs(x64) @ np.abs(wg.astype(np.float64))
    if bias is not None:
        mag = mag + np.abs(bias.astype(np.float64))
    u = 2.0**-24
    return (m + 2) * u * mag + 1e-30


def x_as_f64(x):
    return synth.bf16_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)


def y_to_np(y):
    return y.float().cpu().numpy().astype(np.float64)


def check_routing(L, dbg, T, E, k):
    """Logits within the fp32 bound of the oracle's; top-k, weights and dispatch
    of the oracle recomputed from the GPU's own logits must match bit for bit
    (weights within W_ABS).  Returns the GPU's routing as numpy arrays."""
    lg = dbg["logits"].cpu().numpy()
    ref = oracle.router_logits(L["x"], L["wg"], L["bias"])
    bnd = logit_bound(x_as_f64(L["x"]), L["wg"], L["bias"])
    assert np.all(np.abs(lg.astype(np.float64) - ref.astype(np.float64)) <= bnd), "logits outside fp32 bound"
    idx_g = dbg["topk_idx"].cpu().numpy()
    w_g = dbg["topk_w"].cpu().numpy()
    idx_o, w_o = oracle.topk(lg, k)
    assert np.array_equal(idx_g, idx_o), "top-k differs from the oracle on the GPU's logits"
    assert np.all(np.abs(w_g.astype(np.float64) - w_o.astype(np.float64)) <= W_ABS)
    counts, offsets, perm, _ = oracle.dispatch(idx_g, E)
    assert np.array_equal(dbg["counts"].cpu().numpy(), counts)
    assert np.array_equal(dbg["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(dbg["perm"].cpu().numpy(), perm)
    # end to end: tokens the oracle would route differently from its own logits
    idx_own, _ = oracle.topk(ref, k)
    n_diff = int(np.sum(np.any(idx_own != idx_g, axis=1)))
    return lg, idx_g, w_g, counts, n_diff


def run_layer(L, device="cuda"):
    """GPU forward with every debug output; returns (layer object, y, dbg)."""
    layer = MoELayer(L, device=device)
    dbg = layer.debug_buffers()
    y = layer.forward(dbg=dbg)
    torch.cuda.synchronize()
    return layer, y, dbg
