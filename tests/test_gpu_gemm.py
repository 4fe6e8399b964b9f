"""Parity of the prefill grouped GEMM (MFMA) expert FFN with the CPU oracle.

The layer picks the grouped GEMM for bf16 weights once the experts average
128 rows or more; here it is forced (moe_tuning.ffn_path = MOE_PATH_GEMM) on small shapes so the
oracle finishes in seconds.  The shapes cover reductions of fewer than three
32-k steps (the unpipelined loop) and of many, column counts that leave the
last 256-column block partial, experts with several 256-row blocks, a ragged
last row block, empty experts, one expert holding every row, and expert
sizes just past and just short of whole 256-row blocks.  Bars as in the
other parity tests: max|gpu - oracle| <= 2e-2 max|oracle| + 1e-3.
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


@pytest.fixture(autouse=True)
def _force_gemm(tune):
    tune(ffn_path=M.MOE_PATH_GEMM)


SHAPES = [
    # T, m, p, E, k
    (5, 64, 128, 3, 2),        # up: 2 k-steps (unpipelined); down: 4
    (37, 192, 320, 8, 2),      # 320 columns: partial column block
    (300, 256, 512, 4, 2),     # 150 rows per expert on average, some > 256
    (600, 1024, 1536, 8, 2),   # several row and column blocks
    (1, 512, 384, 16, 2),      # 14 empty experts
    (64, 128, 128, 64, 4),     # 64 experts
    (700, 320, 192, 2, 1),     # 3 row blocks per expert, ragged tail
]


# int4 weights need m and p multiples of 128 (and take 128-row blocks)
SHAPES_I4 = [
    (5, 128, 128, 3, 2),
    (37, 256, 384, 8, 2),      # 384 columns: partial column block
    (300, 256, 512, 4, 2),     # 150 rows per expert on average: two 128-row blocks, ragged
    (600, 1024, 1536, 8, 2),   # several row and column blocks
    (1, 512, 384, 16, 2),      # 14 empty experts
    (64, 128, 128, 64, 4),     # 64 experts
    (700, 384, 256, 2, 1),     # 3 row blocks per expert, ragged tail
]
WEIGHTS = ([("bf16", s) for s in SHAPES] + [("i8", s) for s in SHAPES] + [("fp8", s) for s in SHAPES]
           + [("i4", s) for s in SHAPES_I4])
WIDS = [f"{w}-{'-'.join(map(str, s))}" for w, s in WEIGHTS]


def _routing(T, E, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    return idx, w


@pytest.mark.parametrize("kind", ["swiglu", "relu"])
@pytest.mark.parametrize("wd,shape", WEIGHTS, ids=WIDS)
def test_gemm_expert_ffn_stage(kind, wd, shape):
    T, m, p, E, k = shape
    log(f"gemm expert_ffn kind={kind} w={wd} T={T} m={m} p={p} E={E} k={k}")
    L = synth.make_layer(spec(T, m, p, E, k, kind, wd, seed=7 * T + p, sw=0.05))
    layer = MoELayer(L)
    idx_n, _ = _routing(T, E, k, seed=T + m + 1)
    counts, offsets, perm, _ = oracle.dispatch(idx_n, E)
    y_perm = torch.full((T * k, m), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(layer.handle, layer.x, layer.x_dtype, T, m, p, E, k, to_device(perm), to_device(offsets),
                     y_perm, layer._ws, layer.ws_bytes)
    torch.cuda.synchronize()
    ref, _ = oracle.expert_rows(oracle.Experts.from_layer(L), L["x"], k, perm, offsets)
    got = y_perm.cpu().numpy()
    assert np.all(np.isfinite(got)), "rows left unwritten"
    assert_close(got, ref, wd, "y_perm")
    layer.close()


@pytest.mark.parametrize("kind", ["swiglu", "relu"])
@pytest.mark.parametrize("wd,shape", WEIGHTS, ids=WIDS)
def test_gemm_layer_forward(kind, wd, shape):
    T, m, p, E, k = shape
    log(f"gemm layer_forward kind={kind} w={wd} T={T} m={m} p={p} E={E} k={k}")
    L = synth.make_layer(spec(T, m, p, E, k, kind, wd, seed=T + 3 * E + p, sw=0.05, sr=0.05))
    sp = L["spec"]
    layer = MoELayer(L)
    dbg = layer.debug_buffers()
    y = layer.forward(dbg=dbg)
    torch.cuda.synchronize()
    lg, idx_g, _, counts, _ = check_routing(L, dbg, T, E, k)
    log(f"  counts={counts.tolist()}")
    ref, i_o, _, _ = oracle.forward_tokens(oracle.Experts.from_layer(L), L["x"], L["wg"], L["bias"], sp.k,
                                           np.arange(T), logits=lg)
    assert np.array_equal(i_o, idx_g)
    assert_close(y_to_np(y), ref, wd, "y")
    layer.close()


@pytest.mark.parametrize("wd", ["bf16", "i8", "fp8", "i4"])
def test_gemm_all_rows_on_one_expert(wd):
    """Every token's first choice is expert 3: it holds 600 rows (three or
    five row blocks, the last ragged) while most experts hold none."""
    L = synth.make_layer(spec(600, 256, 384, 16, 2, "swiglu", wd, seed=11))
    L["bias"] = np.zeros(16, np.float32)
    L["bias"][3] = 50.0
    layer = MoELayer(L)
    dbg = layer.debug_buffers()
    y = layer.forward(dbg=dbg)
    torch.cuda.synchronize()
    lg, idx_g, _, counts, _ = check_routing(L, dbg, 600, 16, 2)
    assert counts[3] == 600
    ref, _, _, _ = oracle.forward_tokens(oracle.Experts.from_layer(L), L["x"], L["wg"], L["bias"], 2,
                                         np.arange(600), logits=lg)
    assert_close(y_to_np(y), ref, wd, "y")
    layer.close()


@pytest.mark.parametrize("wd", ["bf16", "i8", "fp8", "i4"])
def test_gemm_repeat_is_bitwise(wd):
    """The GEMM path has no atomics: two calls give identical bits."""
    L = synth.make_layer(spec(300, 256, 512, 4, 2, "swiglu", wd, seed=2))
    layer = MoELayer(L)
    y1 = layer.forward().clone()
    y2 = layer.forward()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    layer.close()


# rows per expert around the 256-row block boundaries: tails of 1, 32, 33,
# 40, 96 and 224 rows after one to eight full blocks, the measured prefill
# layer's 2074, a small and an empty expert
BOUNDARY_COUNTS = [257, 288, 289, 552, 864, 4 * 256 + 224, 8 * 256 + 224, 2074, 5, 0]


@pytest.mark.parametrize("kind", ["swiglu", "relu"])
@pytest.mark.parametrize("wd", ["bf16", "i8"])
def test_gemm_row_block_boundaries(kind, wd):
    """Expert row counts chosen around whole row blocks: every row of every
    expert against the oracle, unwritten rows detected."""
    E, m, p = len(BOUNDARY_COUNTS), 128, 256
    T = sum(BOUNDARY_COUNTS)
    log(f"gemm row-block boundaries kind={kind} w={wd} counts={BOUNDARY_COUNTS}")
    L = synth.make_layer(spec(T, m, p, E, 1, kind, wd, seed=23, sw=0.05))
    layer = MoELayer(L)
    idx_n = np.repeat(np.arange(E, dtype=np.int32), BOUNDARY_COUNTS)
    idx_n = np.random.default_rng(5).permutation(idx_n).reshape(T, 1)
    counts, offsets, perm, _ = oracle.dispatch(idx_n, E)
    assert counts.tolist() == BOUNDARY_COUNTS
    y_perm = torch.full((T, m), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(layer.handle, layer.x, layer.x_dtype, T, m, p, E, 1, to_device(perm), to_device(offsets),
                     y_perm, layer._ws, layer.ws_bytes)
    torch.cuda.synchronize()
    ref, _ = oracle.expert_rows(oracle.Experts.from_layer(L), L["x"], 1, perm, offsets)
    got = y_perm.cpu().numpy()
    assert np.all(np.isfinite(got)), "rows left unwritten"
    assert_close(got, ref, wd, "y_perm")
    layer.close()
