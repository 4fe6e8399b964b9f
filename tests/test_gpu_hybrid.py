"""Parity of the hybrid expert FFN with the CPU oracle.

On bf16 layers with enough rows that some expert may hold more than one
skinny row chunk, experts with at least MOE_HOT_ROWS rows run the grouped
GEMM on a second stream while the skinny kernels serve the rest on the
caller's stream; both add into the same fp32 output.  These tests force the
path (MOE_FFN_PATH=h) with small thresholds on skewed (Zipf) and
one-hot-expert routings, for the fused layer and for the expert-FFN stage
(unweighted rows), at the bars of the other parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import mixture_experts_layer_gemv_amd as M
from mixture_experts_layer_gemv_amd.layer import MoELayer, to_device

from _gpu import assert_close, check_routing, log, spec, y_to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()
    yield
    torch.cuda.synchronize()


CASES = [
    # T, m, p, E, k, zipf, hot rows
    (200, 256, 512, 8, 2, 1.2, 40),
    (300, 512, 384, 16, 2, 1.2, 24),
    (96, 128, 256, 4, 2, None, 30),
    (257, 320, 192, 8, 1, 1.5, 17),
    (150, 256, 320, 64, 4, 1.2, 20),
]


@pytest.mark.parametrize("kind", ["swiglu", "relu"])
@pytest.mark.parametrize("T,m,p,E,k,zipf,hot", CASES)
def test_hybrid_layer_forward(kind, T, m, p, E, k, zipf, hot, monkeypatch):
    monkeypatch.setenv("MOE_FFN_PATH", "h")
    monkeypatch.setenv("MOE_HOT_ROWS", str(hot))
    log(f"hybrid layer kind={kind} T={T} m={m} p={p} E={E} k={k} zipf={zipf} hot>={hot}")
    L = synth.make_layer(spec(T, m, p, E, k, kind, "bf16", seed=T + p + E, zipf=zipf, sw=0.05, sr=0.05))
    layer = MoELayer(L)
    dbg = layer.debug_buffers()
    y = layer.forward(dbg=dbg)
    torch.cuda.synchronize()
    lg, idx_g, _, counts, _ = check_routing(L, dbg, T, E, k)
    log(f"  counts={counts.tolist()} hot experts={int(np.sum(counts >= hot))}")
    ref, i_o, _, _ = oracle.forward_tokens(oracle.Experts.from_layer(L), L["x"], L["wg"], L["bias"], k,
                                           np.arange(T), logits=lg)
    assert np.array_equal(i_o, idx_g)
    assert_close(y_to_np(y), ref, "bf16", "y")
    layer.close()


@pytest.mark.parametrize("T,m,p,E,k,zipf,hot", CASES[:3])
def test_hybrid_expert_ffn_stage(T, m, p, E, k, zipf, hot, monkeypatch):
    monkeypatch.setenv("MOE_FFN_PATH", "h")
    monkeypatch.setenv("MOE_HOT_ROWS", str(hot))
    L = synth.make_layer(spec(T, m, p, E, k, "swiglu", "bf16", seed=5 * T + p, sw=0.05))
    layer = MoELayer(L)
    rng = np.random.default_rng(T + m)
    # skewed routing: expert 0 takes every token's first choice
    idx = np.stack([np.concatenate([[0], 1 + rng.permutation(E - 1)[:k - 1]]) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, _ = oracle.dispatch(idx, E)
    log(f"hybrid expert_ffn counts={counts.tolist()} hot>={hot}")
    y_perm = torch.full((T * k, m), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(layer.handle, layer.x, layer.x_dtype, T, m, p, E, k, to_device(perm), to_device(offsets),
                     y_perm, layer._ws, layer.ws_bytes)
    torch.cuda.synchronize()
    ref, _ = oracle.expert_rows(oracle.Experts.from_layer(L), L["x"], k, perm, offsets)
    got = y_perm.cpu().numpy()
    assert np.all(np.isfinite(got)), "rows left unwritten"
    assert_close(got, ref, "bf16", "y_perm")
    layer.close()


@pytest.mark.parametrize("ksplit", ["1", "4"])
def test_hybrid_repeat(ksplit, monkeypatch):
    """Without a split reduction each output element is the sum of two fp32
    products (top-2) added onto zero, the same bits in either order whichever
    stream adds first; with the hot experts' down projection split into four
    slices only the order of the atomic adds may differ."""
    monkeypatch.setenv("MOE_FFN_PATH", "h")
    monkeypatch.setenv("MOE_HOT_ROWS", "40")
    monkeypatch.setenv("MOE_GEMM_KSPLIT", ksplit)
    L = synth.make_layer(spec(200, 256, 512, 8, 2, seed=8, zipf=1.2))
    layer = MoELayer(L)
    y1 = layer.forward().clone()
    for _ in range(3):
        y2 = layer.forward()
        torch.cuda.synchronize()
        if ksplit == "1":
            assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
        else:
            a, b = y_to_np(y1), y_to_np(y2)
            assert np.max(np.abs(a - b)) <= 2.0**-7 * np.max(np.abs(a))
    layer.close()
