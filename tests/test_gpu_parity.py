"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Routing indices, counts, offsets and permutations are compared bit for bit
(the oracle re-ranks the GPU's own fp32 logits); logits within the fp32
dot-product bound; gate weights within 2e-6; expert and layer outputs within
max|gpu - oracle| <= 2e-2 max|oracle| + 1e-3 (bf16 / int8 weights) or
1e-4 max|oracle| (fp32 layers).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import mixture_experts_layer_gemv_amd as M
from mixture_experts_layer_gemv_amd.layer import MoELayer, to_device

from _gpu import W_ABS, assert_close, check_routing, log, logit_bound, spec, x_as_f64, y_to_np

pytestmark = pytest.mark.gpu

DT = {"f32": M.MOE_F32, "bf16": M.MOE_BF16, "i8": M.MOE_I8}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# routing stage
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,m,E,k,zipf", [(1, 64, 1, 1, None), (5, 128, 3, 2, None), (70, 256, 8, 2, None),
                                          (33, 4096, 8, 2, None), (129, 512, 16, 2, 1.2), (40, 192, 33, 3, None),
                                          (19, 320, 64, 4, 1.2), (8, 64, 8, 8, None),
                                          # the shapes for a few hundred and for past 1024 tokens
                                          # (ragged last blocks)
                                          (300, 1024, 8, 2, None), (1500, 4096, 8, 2, None),
                                          (1027, 4096, 16, 4, 1.2)])
def test_route_topk(x_dtype, T, m, E, k, zipf):
    log(f"route_topk x={x_dtype} T={T} m={m} E={E} k={k} zipf={zipf}")
    sp = synth.LayerSpec("r", T, m, 64, E, k, "swiglu", x_dtype, "bf16", seed=T + E, sigma_router=0.05, zipf_s=zipf)
    L = synth.make_layer(sp, with_weights=False)
    x, wg, b = to_device(L["x"]), to_device(L["wg"]), to_device(L["bias"])
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    M.moe_route_topk(x, DT[x_dtype], wg, b, T, m, E, k, 0, lg, idx, w)
    torch.cuda.synchronize()
    lg_n = lg.cpu().numpy()
    ref = oracle.router_logits(L["x"], L["wg"], L["bias"])
    assert np.all(np.abs(lg_n.astype(np.float64) - ref) <= logit_bound(x_as_f64(L["x"]), L["wg"], L["bias"]))
    i_o, w_o = oracle.topk(lg_n, k)
    assert np.array_equal(idx.cpu().numpy(), i_o)
    assert np.all(np.abs(w.cpu().numpy().astype(np.float64) - w_o) <= W_ABS)
    # logits may be omitted
    idx2 = torch.empty_like(idx)
    M.moe_route_topk(x, DT[x_dtype], wg, b, T, m, E, k, 0, None, idx2, w)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)


CRAFTED = [
    [0.5] * 8,
    [1.0, 2.0, 2.0, 1.0, -1.0, 2.0, 0.0, -0.0],
    [0.0, -0.0, -0.0, 0.0, -1.0, -1.0, -2.0, -3.0],
    [-math.inf, 3.0, math.inf, math.inf, -1.0, 0.0, 1.0, 2.0],
    [math.nan, 1.0, math.nan, -math.inf, -math.inf, 5.0, math.nan, 0.0],
    [math.nan] * 7 + [1.0],
    [math.nan] * 8,
    [-math.inf] * 8,
    [3.0, 1e-30, -1e-30, 3.0, float(np.nextafter(np.float32(3.0), np.float32(0))), 0.0, 2.0, 1.0],
]


@pytest.mark.parametrize("k", [1, 2, 3, 8])
def test_route_topk_crafted_logits(k):
    """Ties, signed zeros, infinities and NaN through MOE_ROUTE_LOGITS_IN."""
    log(f"route_topk crafted k={k}")
    lg_n = np.array(CRAFTED, np.float32)
    rng = np.random.default_rng(k)
    lg_n = np.concatenate([lg_n, rng.integers(-2, 3, size=(60, 8)).astype(np.float32)])
    T, E = lg_n.shape
    lg = to_device(lg_n)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    M.moe_route_topk(None, M.MOE_F32, None, None, T, 64, E, k, M.MOE_ROUTE_LOGITS_IN, lg, idx, w)
    torch.cuda.synchronize()
    i_o, w_o = oracle.topk(lg_n, k)
    assert np.array_equal(idx.cpu().numpy(), i_o)
    w_g = w.cpu().numpy()
    assert np.array_equal(np.isnan(w_g), np.isnan(w_o))
    ok = ~np.isnan(w_o)
    assert np.all(np.abs(w_g[ok].astype(np.float64) - w_o[ok]) <= W_ABS)


# ---------------------------------------------------------------------------
# dispatch stage
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k,mode", [(1, 1, 1, "rand"), (1, 8, 2, "rand"), (31, 8, 2, "rand"),
                                        (32, 8, 2, "rand"), (512, 8, 2, "rand"), (513, 8, 2, "rand"),
                                        (300, 64, 4, "rand"), (8192, 8, 2, "rand"), (20000, 16, 2, "zipf"),
                                        (777, 3, 3, "rand"), (1000, 16, 2, "one"), (50, 64, 1, "sparse")])
def test_dispatch(T, E, k, mode):
    log(f"dispatch T={T} E={E} k={k} mode={mode}")
    rng = np.random.default_rng(T * 7 + E)
    if mode == "one":
        idx_n = np.zeros((T, k), np.int32)
        idx_n[:, 0] = 5
        idx_n[:, 1:] = rng.integers(0, E, size=(T, k - 1))
    elif mode == "zipf":
        p = np.exp(synth.zipf_logit_bias(E, 1.2).astype(np.float64))
        idx_n = rng.choice(E, size=(T, k), p=p / p.sum()).astype(np.int32)
    elif mode == "sparse":
        idx_n = rng.integers(60, 64, size=(T, k)).astype(np.int32)
    else:
        idx_n = rng.integers(0, E, size=(T, k)).astype(np.int32)
    n = T * k
    idx = to_device(idx_n)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(n, dtype=torch.int32, device="cuda")
    inv = torch.empty(n, dtype=torch.int32, device="cuda")
    M.moe_dispatch(idx, T, E, k, counts, offsets, perm, inv)
    torch.cuda.synchronize()
    c, o, p_, iv = oracle.dispatch(idx_n, E)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(perm.cpu().numpy(), p_)
    assert np.array_equal(inv.cpu().numpy(), iv)


# ---------------------------------------------------------------------------
# expert FFN and combine stages
# ---------------------------------------------------------------------------

SHAPES = [
    # T, m, p, E, k
    (5, 64, 128, 3, 2),
    (37, 192, 320, 8, 2),
    (24, 2048, 1600, 4, 2),
    (64, 128, 128, 64, 4),
    (9, 128, 64, 8, 8),
    (17, 256, 256, 1, 1),
    (1, 512, 384, 16, 2),
    (257, 256, 512, 16, 2),
]
KINDS = [("swiglu", "bf16"), ("relu", "bf16"), ("swiglu", "i8"), ("relu", "i8"), ("swiglu", "f32"), ("relu", "f32")]


def _routing(T, E, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    return idx, w


@pytest.mark.parametrize("kind,w_dtype", KINDS)
@pytest.mark.parametrize("T,m,p,E,k", SHAPES)
def test_expert_ffn_stage(kind, w_dtype, T, m, p, E, k):
    log(f"expert_ffn kind={kind} w={w_dtype} T={T} m={m} p={p} E={E} k={k}")
    sp = spec(T, m, p, E, k, kind, w_dtype, seed=3 * T + p, sw=0.05)
    L = synth.make_layer(sp)
    layer = MoELayer(L)
    idx_n, _ = _routing(T, E, k, seed=T + m)
    counts, offsets, perm, inv = oracle.dispatch(idx_n, E)
    y_perm = torch.empty((T * k, m), dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(layer.handle, layer.x, layer.x_dtype, T, m, p, E, k, to_device(perm), to_device(offsets),
                     y_perm, layer._ws, layer.ws_bytes)
    torch.cuda.synchronize()
    ref, _ = oracle.expert_rows(oracle.Experts.from_layer(L), L["x"], k, perm, offsets)
    assert_close(y_perm.cpu().numpy(), ref, w_dtype, "y_perm")
    layer.close()


@pytest.mark.parametrize("y_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,m,k,E", [(1, 64, 1, 1), (33, 192, 2, 8), (300, 512, 4, 16), (7, 4096, 8, 8)])
def test_combine_stage(y_dtype, T, m, k, E):
    log(f"combine y={y_dtype} T={T} m={m} k={k}")
    idx_n, w_n = _routing(T, E, k, seed=m + k)
    _, _, perm, inv = oracle.dispatch(idx_n, E)
    rng = np.random.default_rng(T)
    yp = rng.normal(size=(T * k, m)).astype(np.float32)
    y = torch.empty((T, m), dtype=torch.float32 if y_dtype == "f32" else torch.bfloat16, device="cuda")
    M.moe_combine(to_device(yp), to_device(inv), to_device(w_n), T, m, k, y, DT[y_dtype])
    torch.cuda.synchronize()
    ref = oracle.combine(yp.astype(np.float64), inv, idx_n, w_n)
    got = y_to_np(y)
    if y_dtype == "f32":
        assert np.max(np.abs(got - ref)) <= 1e-6 * max(1.0, np.max(np.abs(ref)))
    else:  # one bf16 rounding of the fp32 sum
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0**-8 + 1e-6)


# ---------------------------------------------------------------------------
# the fused layer
# ---------------------------------------------------------------------------

def _layer_case(L, sample=None, seed=0):
    sp = L["spec"]
    layer = MoELayer(L)
    dbg = layer.debug_buffers()
    y = layer.forward(dbg=dbg)
    torch.cuda.synchronize()
    lg, idx_g, w_g, counts, n_diff = check_routing(L, dbg, sp.T, sp.E, sp.k)
    log(f"  counts={counts.tolist()} tokens routed differently from oracle logits: {n_diff}")
    tokens = np.arange(sp.T) if sample is None else np.sort(
        np.random.default_rng(seed).choice(sp.T, size=min(sample, sp.T), replace=False))
    X = oracle.Experts.from_layer(L)
    ref, i_o, w_o, _ = oracle.forward_tokens(X, L["x"], L["wg"], L["bias"], sp.k, tokens, logits=lg)
    assert np.array_equal(i_o, idx_g[tokens])
    got = y_to_np(y)[tokens]
    assert_close(got, ref, sp.w_dtype, f"y[{len(tokens)} tokens]")
    return layer, y, dbg


@pytest.mark.parametrize("kind,w_dtype", KINDS)
@pytest.mark.parametrize("T,m,p,E,k", SHAPES + [(200, 256, 256, 8, 2)])
def test_layer_forward(kind, w_dtype, T, m, p, E, k):
    zipf = 1.2 if T == 200 else None
    log(f"layer_forward kind={kind} w={w_dtype} T={T} m={m} p={p} E={E} k={k} zipf={zipf}")
    L = synth.make_layer(spec(T, m, p, E, k, kind, w_dtype, seed=T + E + p, zipf=zipf, sw=0.05, sr=0.05))
    layer, _, _ = _layer_case(L)
    layer.close()


@pytest.mark.parametrize("w_dtype", ["bf16", "i8", "f32"])
def test_layer_all_tokens_one_expert(w_dtype):
    """A router bias that sends every token's first choice to expert 3 (one
    expert holds T rows, several experts hold none)."""
    log(f"all-on-one w={w_dtype}")
    L = synth.make_layer(spec(150, 256, 320, 16, 2, "swiglu", w_dtype, seed=5))
    L["bias"] = np.zeros(16, np.float32)
    L["bias"][3] = 50.0
    layer, _, dbg = _layer_case(L)
    assert dbg["counts"][3].item() == 150
    layer.close()


def test_layer_T0_is_noop():
    L = synth.make_layer(spec(4, 64, 64, 4, 2))
    layer = MoELayer(L)
    y = torch.full((1, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    M.moe_layer_forward(layer.handle, layer.wg, None, layer.x, layer.x_dtype, 0, 64, 64, 4, 2, y, M.MOE_BF16,
                        layer._ws, layer.ws_bytes)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    layer.close()


def test_layer_workspace_too_small():
    L = synth.make_layer(spec(4, 64, 64, 4, 2))
    layer = MoELayer(L)
    y = layer.new_output()
    with pytest.raises(M.MoeError) as ei:
        M.moe_layer_forward(layer.handle, layer.wg, None, layer.x, layer.x_dtype, 4, 64, 64, 4, 2, y, M.MOE_BF16,
                            layer._ws, layer.ws_bytes - 1)
    assert ei.value.status == M.MOE_ERR_WORKSPACE
    with pytest.raises(M.MoeError) as ei:
        M.moe_layer_forward(layer.handle, layer.wg, None, layer.x, layer.x_dtype, 4, 64, 128, 4, 2, y, M.MOE_BF16,
                            layer._ws, layer.ws_bytes)
    assert ei.value.status == M.MOE_ERR_INVALID_ARG
    layer.close()


@pytest.mark.parametrize("ksplit", ["1", "4"])
def test_layer_repeat_is_deterministic(ksplit, tune):
    """Routing repeats bit for bit.  Without a split reduction the top-2
    combine adds two terms onto zero, so the output repeats bit for bit too;
    with one, only the order of fp32 atomic adds may differ."""
    tune(down_ksplit=int(ksplit))
    L = synth.make_layer(spec(64, 512, 256, 8, 2, seed=9))
    layer = MoELayer(L)
    d1, d2 = layer.debug_buffers(), layer.debug_buffers()
    y1 = layer.forward(dbg=d1).clone()
    y2 = layer.forward(dbg=d2)
    torch.cuda.synchronize()
    for key in d1:
        assert torch.equal(d1[key], d2[key]), key
    if ksplit == "1":
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    else:
        a, b = y_to_np(y1), y_to_np(y2)
        assert np.max(np.abs(a - b)) <= 2.0**-7 * np.max(np.abs(a))
    layer.close()


def test_layer_smaller_batch_reuses_handle():
    """One weights handle serves calls with different T."""
    L = synth.make_layer(spec(48, 256, 256, 8, 2, seed=4))
    layer = MoELayer(L)
    X = oracle.Experts.from_layer(L)
    for T in (48, 5, 1, 30):
        dbg = layer.debug_buffers(T)
        y = layer.forward(x=layer.x[:T].contiguous(), T=T, dbg=dbg)
        torch.cuda.synchronize()
        lg = dbg["logits"].cpu().numpy()
        ref, _, _, _ = oracle.forward_tokens(X, L["x"][:T], L["wg"], None, 2, np.arange(T), logits=lg)
        assert_close(y_to_np(y), ref, "bf16", f"T={T}")
    layer.close()
