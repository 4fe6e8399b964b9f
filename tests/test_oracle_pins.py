"""Pins of the CPU oracle against facts fixed outside it.

Each test ties one part of the oracle to something it does not compute
itself: a closed form the pages print, a hand-worked example, a brute-force
enumeration, an invariant, or an independent library routine (torch fp64).
"""
import itertools
import json
import dataclasses
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _layer(syn, T, m, p, E, k, kind, w_dtype, seed, x_dtype=None, zipf=None, sw=0.05, sr=0.05):
    x_dtype = x_dtype or ("f32" if w_dtype == "f32" else "bf16")
    sp = syn.LayerSpec("t", T, m, p, E, k, kind, x_dtype, w_dtype, seed, sigma_router=sr, sigma_w=sw, zipf_s=zipf)
    return syn.make_layer(sp)


def _to64(syn, a):
    if a.dtype == np.uint16:
        return syn.bf16_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


# --------------------------------------------------------------------------
# closed forms printed on the pages: |O| and |E|
# --------------------------------------------------------------------------

def test_op_count_matches_printed_formula_relu(orc, syn):
    """|O| = q*p*(2m-1) + q*m*(2p-1) (HARMOEny article, section 3.2), exact, at the tiny fp32 layer."""
    L = syn.make_layer(syn.spec("c1"))
    X = orc.Experts.from_layer(L)
    r = orc.layer_forward(X, L["x"], L["wg"], L["bias"], 2)
    q, m, p = 32 * 2, 256, 512
    assert int(r["ops"][0]) == q * p * (2 * m - 1) + q * m * (2 * p - 1) == 33_505_280
    assert int(r["ops"][1]) == q * p  # one ReLU per hidden unit


@pytest.mark.parametrize("q_rows", [1, 3, 7])
def test_op_count_swiglu_form(orc, syn, q_rows):
    """SwiGLU adds a second m x p dot-product bank: 2qp(2m-1) + qm(2p-1), plus qp SiLU and qp products."""
    L = _layer(syn, 5, 24, 40, 4, 2, "swiglu", "bf16", 11)
    X = orc.Experts.from_layer(L)
    r = orc.layer_forward(X, L["x"], L["wg"], None, 2)
    rows = np.arange(q_rows, dtype=np.int32)
    _, ops = orc.expert_rows(X, L["x"], 2, r["perm"], r["offsets"], rows)
    m, p = 24, 40
    assert int(ops[0]) == 2 * q_rows * p * (2 * m - 1) + q_rows * m * (2 * p - 1)
    assert int(ops[1]) == q_rows * p and int(ops[2]) == q_rows * p


def test_param_bytes_printed_formula_and_page_sizes(orc, syn):
    """|E| = (mp + pm) * dtype at the tiny layer; SwiGLU 3*m*p*2 B against the printed expert sizes."""
    figs = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    L = syn.make_layer(syn.spec("c1"))
    X = orc.Experts.from_layer(L)
    assert X.param_bytes() == (256 * 512 + 512 * 256) * 4 == 1_048_576
    assert L["w1"][0].nbytes + L["w2"][0].nbytes == X.param_bytes()
    # Mixtral-8x7B expert: SwiGLU, m=4096, p=14336, bf16 -> 352,321,536 B = 336 MiB ~ "340 MB"
    mix = syn.spec("c2")
    assert mix.expert_bytes() == 352_321_536
    assert abs(mix.expert_bytes() / 2**20 - figs["mixtral_expert_mb"]["value"]) / 340 < 0.02
    assert mix.E == figs["mixtral_experts_per_layer"]["value"]
    # Phi-3.5-MoE expert: m=4096, p=6400 -> 157,286,400 B, within 4% of "152 MB"
    phi = syn.spec("c3")
    assert abs(phi.expert_bytes() / 1e6 - figs["phi35_expert_mb"]["value"]) / 152 < 0.04
    assert phi.E == figs["phi35_experts_per_layer"]["value"]


def test_prefetch_threshold_algebra():
    """q > phi*dtype/(2 beta) follows from |O|/phi > |E|/beta with |O| ~ 4qmp (HARMOEny article, section 3.2)."""
    m, p, dtype = 4096, 14336, 2
    for phi, beta in [(2.5e15, 8e12), (1.65e14, 2.5e10), (1e12, 1e9)]:
        q_star = phi * dtype / (2 * beta)
        exact = lambda q: q * p * (2 * m - 1) + q * m * (2 * p - 1)
        E_bytes = (m * p + p * m) * dtype
        # just above the threshold compute covers the load, just below it does not
        assert exact(math.ceil(q_star * 1.001)) / phi > E_bytes / beta
        assert exact(math.floor(q_star * 0.999)) / phi < E_bytes / beta


# --------------------------------------------------------------------------
# hand-worked examples
# --------------------------------------------------------------------------

def _hand_relu_experts(orc):
    # expert 0: W1 = [[1,-1],[0,2]], W2 = [[1,0],[2,1]];  expert 1: W1 = [[2,0],[1,1]], W2 = [[0,1],[1,-1]]
    w1 = np.array([[[1, -1], [0, 2]], [[2, 0], [1, 1]]], np.float32)
    w2 = np.array([[[1, 0], [2, 1]], [[0, 1], [1, -1]]], np.float32)
    return orc.Experts("relu", w1, w2)


def test_hand_worked_relu_top1(orc):
    """x0 = [1,2] -> expert 1: relu([4,2]) W2 = [2,2];  x1 = [2,-1] -> expert 0: relu([2,-4]) W2 = [2,0]."""
    X = _hand_relu_experts(orc)
    x = np.array([[1, 2], [2, -1]], np.float32)
    wg = np.eye(2, dtype=np.float32)
    r = orc.layer_forward(X, x, wg, None, 1)
    assert r["idx"].tolist() == [[1], [0]]
    assert r["w"].tolist() == [[1.0], [1.0]]
    assert r["y"].tolist() == [[2.0, 2.0], [2.0, 0.0]]
    assert r["counts"].tolist() == [1, 1] and r["perm"].tolist() == [1, 0]


def test_hand_worked_relu_top2(orc):
    """Token [1,2] with logits [1,2]: w = [1/(1+e^-1), e^-1/(1+e^-1)] on experts (1, 0); expert 0 gives [7,3]."""
    X = _hand_relu_experts(orc)
    x = np.array([[1, 2]], np.float32)
    r = orc.layer_forward(X, x, np.eye(2, dtype=np.float32), None, 2)
    w_hi = np.float32(1.0 / (1.0 + math.exp(-1.0)))
    w_lo = np.float32(math.exp(-1.0) / (1.0 + math.exp(-1.0)))
    assert r["idx"].tolist() == [[1, 0]]
    assert r["w"][0].tolist() == [w_hi, w_lo]
    want = [float(w_lo) * 7 + float(w_hi) * 2, float(w_lo) * 3 + float(w_hi) * 2]  # ascending expert order
    assert r["y"][0].tolist() == want


def test_hand_worked_swiglu_and_silu_points(orc):
    """g = [1,-1], u = [2,-3]: h = [2 SiLU(1), -3 SiLU(-1)]; o = h W2 with W2 = [[1,1],[0,2]]."""
    w1 = np.eye(2, dtype=np.float32)[None]
    w3 = np.array([[[2, 0], [0, 3]]], np.float32)
    w2 = np.array([[[1, 1], [0, 2]]], np.float32)
    X = orc.Experts("swiglu", w1, w2, w3)
    o, ops = orc.expert_apply(X, 0, np.array([1.0, -1.0]))
    silu1, silum1 = 0.7310585786300049, -0.2689414213699951  # 1/(1+e^-1), -1/(1+e)
    h = [2 * silu1, -3 * silum1]
    assert o[0] == pytest.approx(h[0], rel=1e-15)
    assert o[1] == pytest.approx(h[0] + 2 * h[1], rel=1e-15)
    # SiLU(0) = 0 and the ReLU form on a 1x1 expert
    Xs = orc.Experts("swiglu", np.ones((1, 1, 1), np.float32), np.ones((1, 1, 1), np.float32),
                     np.ones((1, 1, 1), np.float32))
    assert orc.expert_apply(Xs, 0, np.array([0.0]))[0][0] == 0.0
    Xr = orc.Experts("relu", np.ones((1, 1, 1), np.float32), np.ones((1, 1, 1), np.float32))
    assert orc.expert_apply(Xr, 0, np.array([-3.0]))[0][0] == 0.0
    assert orc.expert_apply(Xr, 0, np.array([2.5]))[0][0] == 2.5


# --------------------------------------------------------------------------
# router: library special case (torch fp64 matmul)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("with_bias", [False, True])
def test_router_logits_vs_torch_fp64(orc, syn, x_dtype, with_bias):
    L = _layer(syn, 37, 96, 64, 12, 2, "swiglu", "bf16", 3, x_dtype=x_dtype, zipf=1.2 if with_bias else None)
    lg = orc.router_logits(L["x"], L["wg"], L["bias"])
    ref = torch.from_numpy(_to64(syn, L["x"])) @ torch.from_numpy(L["wg"].astype(np.float64))
    if with_bias:
        ref = ref + torch.from_numpy(L["bias"].astype(np.float64))
    ref32 = ref.float().numpy()
    # both round a double sum to fp32; the double sums differ only in order
    assert np.all(np.abs(lg.astype(np.float64) - ref32.astype(np.float64)) <= np.spacing(np.abs(ref32)))


# --------------------------------------------------------------------------
# top-k: brute force over subsets, crafted ties and non-finite values
# --------------------------------------------------------------------------

def _before(va, a, vb, b):
    """Ranking used by the oracle, restated: numbers before NaN, larger first, lower index on ties."""
    if math.isnan(va) or math.isnan(vb):
        return (a < b) if (math.isnan(va) and math.isnan(vb)) else math.isnan(vb)
    return va > vb or (va == vb and a < b)


def _brute_topk(row, k):
    E = len(row)
    winners = [S for S in itertools.combinations(range(E), k)
               if all(_before(row[a], a, row[b], b) for a in S for b in range(E) if b not in S)]
    assert len(winners) == 1
    S = list(winners[0])
    # slot order: each slot ranks before every later one
    return sorted(S, key=lambda a: sum(_before(row[b], b, row[a], a) for b in S))


CRAFTED = [
    [0.5, 0.5, 0.5, 0.5, 0.5, 0.5, 0.5, 0.5],
    [1.0, 2.0, 2.0, 1.0, -1.0, 2.0, 0.0, -0.0],
    [0.0, -0.0, -0.0, 0.0, -1.0, -1.0, -2.0, -3.0],
    [-math.inf, 3.0, math.inf, math.inf, -1.0, 0.0, 1.0, 2.0],
    [math.nan, 1.0, math.nan, -math.inf, -math.inf, 5.0, math.nan, 0.0],
    [math.nan, math.nan, math.nan, math.nan, math.nan, math.nan, math.nan, 1.0],
    [math.nan] * 8,
    [-math.inf] * 8,
    [3.0, 1e-30, -1e-30, 3.0, float(np.nextafter(np.float32(3.0), np.float32(0))), 0.0, 2.0, 1.0],
]


@pytest.mark.parametrize("k", [1, 2, 3, 8])
def test_topk_crafted_rows_brute_force(orc, k):
    logits = np.array(CRAFTED, np.float32)
    idx, w = orc.topk(logits, k)
    for t, row in enumerate(logits.tolist()):
        assert idx[t].tolist() == _brute_topk(row, k), (t, row)


@pytest.mark.parametrize("E,k", [(1, 1), (3, 2), (8, 2), (8, 8), (16, 2), (64, 4)])
def test_topk_random_vs_stable_lexsort(orc, E, k):
    rng = np.random.default_rng(E * 100 + k)
    # few distinct values, so ties are common
    logits = rng.integers(-3, 4, size=(200, E)).astype(np.float32) * np.float32(0.25)
    idx, _ = orc.topk(logits, k)
    ref = np.stack([np.lexsort((np.arange(E), -row))[:k] for row in logits])
    assert np.array_equal(idx, ref)


def test_gate_weight_closed_forms(orc):
    rng = np.random.default_rng(5)
    logits = rng.normal(size=(64, 8)).astype(np.float32)
    idx1, w1 = orc.topk(logits, 1)
    assert np.all(w1 == 1.0)
    idx2, w2 = orc.topk(logits, 2)
    for t in range(64):
        l0, l1 = float(logits[t, idx2[t, 0]]), float(logits[t, idx2[t, 1]])
        assert w2[t, 0] == np.float32(1.0 / (1.0 + math.exp(l1 - l0)))
        assert abs(float(w2[t, 0]) + float(w2[t, 1]) - 1.0) < 1e-7
    _, we = orc.topk(np.full((3, 8), 0.7, np.float32), 4)
    assert np.all(we == np.float32(0.25))
    # same as a full softmax over E renormalised over the selected k (torch, fp64)
    idx3, w3 = orc.topk(logits, 3)
    sm = torch.softmax(torch.from_numpy(logits.astype(np.float64)), dim=1).numpy()
    sel = np.take_along_axis(sm, idx3, 1)
    assert np.allclose(w3, sel / sel.sum(1, keepdims=True), rtol=1e-6, atol=0)


def test_gate_weights_nonfinite(orc):
    lg = np.array([[math.nan, 1.0, 0.0], [math.inf, 1.0, 0.0], [-math.inf, -math.inf, -math.inf]], np.float32)
    idx, w = orc.topk(lg, 2)
    assert idx.tolist() == [[1, 2], [0, 1], [0, 1]]
    assert w[0, 0] == np.float32(1 / (1 + math.exp(-1)))
    assert np.isnan(w[1]).all() and np.isnan(w[2]).all()  # inf - inf in the exponent
    idx, w = orc.topk(lg, 3)
    assert idx[0].tolist() == [1, 2, 0] and np.isnan(w[0]).all()  # a selected NaN poisons the softmax


# --------------------------------------------------------------------------
# dispatch: invariants, brute force, library special case
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k", [(0, 4, 1), (1, 1, 1), (7, 3, 2), (64, 8, 2), (257, 16, 2), (100, 64, 4),
                                   (33, 5, 5)])
def test_dispatch_invariants_and_brute_force(orc, T, E, k):
    rng = np.random.default_rng(T + E + k)
    if T:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    else:
        idx = np.zeros((0, k), np.int32)
    counts, offsets, perm, inv = orc.dispatch(idx, E)
    flat = idx.reshape(-1)
    n = T * k
    assert counts.sum() == n and offsets[0] == 0 and offsets[E] == n
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(perm), np.arange(n))
    assert np.all(np.diff(flat[perm]) >= 0) if n else True
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0) and np.all(flat[seg] == e)
    assert np.array_equal(inv[perm], np.arange(n))
    brute = [a for e in range(E) for a in range(n) if flat[a] == e]
    assert perm.tolist() == brute
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(counts, np.bincount(flat, minlength=E))


def test_dispatch_rejects_out_of_range(orc):
    with pytest.raises(ValueError):
        orc.dispatch(np.array([[0], [4]], np.int32), 4)


# --------------------------------------------------------------------------
# routed = dense masked brute force (bit-identical in double)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kind,w_dtype", [("relu", "f32"), ("swiglu", "f32"), ("swiglu", "bf16"),
                                          ("relu", "bf16"), ("swiglu", "i8")])
@pytest.mark.parametrize("E,k", [(1, 1), (3, 2), (8, 1), (8, 2), (8, 8)])
def test_routed_equals_dense_masked(orc, syn, kind, w_dtype, E, k):
    L = _layer(syn, 8, 32, 64, E, k, kind, w_dtype, seed=E * 10 + k)
    X = orc.Experts.from_layer(L)
    r = orc.layer_forward(X, L["x"], L["wg"], None, k)
    yd = orc.dense_masked(X, L["x"], r["idx"], r["w"])
    assert np.array_equal(r["y"], yd)
    ys, _, _, _ = orc.forward_tokens(X, L["x"], L["wg"], None, k, np.arange(8)[::-1])
    assert np.array_equal(ys, r["y"][::-1])


# --------------------------------------------------------------------------
# the MLP itself: E=1, k=1 against the torch fp64 chain
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kind,w_dtype", [("relu", "f32"), ("relu", "bf16"), ("swiglu", "f32"),
                                          ("swiglu", "bf16"), ("swiglu", "i8"), ("relu", "i8"),
                                          ("swiglu", "i4"), ("relu", "i4")])
def test_single_expert_is_dense_mlp(orc, syn, kind, w_dtype):
    L = _layer(syn, 9, 48, 80, 1, 1, kind, w_dtype, seed=77)
    X = orc.Experts.from_layer(L)
    r = orc.layer_forward(X, L["x"], L["wg"], None, 1)
    assert np.all(r["w"] == 1.0)

    def deq(key):
        w = L[key][0]
        if w_dtype in ("i8", "i4"):
            return torch.from_numpy(w.astype(np.float64) * L["s" + key[1:]][0].astype(np.float64)[None, :])
        return torch.from_numpy(_to64(syn, w))

    x = torch.from_numpy(_to64(syn, L["x"]))
    if kind == "relu":
        ref = torch.relu(x @ deq("w1")) @ deq("w2")
    else:
        ref = (torch.nn.functional.silu(x @ deq("w1")) * (x @ deq("w3"))) @ deq("w2")
    assert np.allclose(r["y"], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_int8_quantisation_closed_forms(syn):
    """Per output channel: max|q| = 127 and |W - q s| <= s/2, with W redrawn from the same stream."""
    E, K, N = 2, 64, 48
    q, s = syn.int8_quant(9, syn.TID_W1, 0.02, E, K, N)
    W = syn.normal_f32(9, syn.TID_W1, 0.02, (E, K, N)).astype(np.float64)
    assert np.all(np.abs(q).max(axis=1) == 127)
    err = np.abs(W - q.astype(np.float64) * s[:, None, :].astype(np.float64))
    assert np.all(err <= s[:, None, :].astype(np.float64) / 2 * (1 + 1e-6))


def test_int4_quantisation_closed_forms(syn):
    """The int4 rule: per output channel s = max|W| / 7, max|q| = 7, q in [-7, 7] and |W - q s| <= s/2."""
    E, K, N = 2, 64, 48
    q, s = syn.int4_quant(9, syn.TID_W1, 0.02, E, K, N)
    W = syn.normal_f32(9, syn.TID_W1, 0.02, (E, K, N)).astype(np.float64)
    assert q.dtype == np.int8 and q.min() >= -7 and q.max() <= 7
    assert np.all(np.abs(q).max(axis=1) == 7)
    assert np.allclose(s, (np.abs(W).max(axis=1) / 7).astype(np.float32), rtol=0, atol=0)
    err = np.abs(W - q.astype(np.float64) * s[:, None, :].astype(np.float64))
    assert np.all(err <= s[:, None, :].astype(np.float64) / 2 * (1 + 1e-6))


# --------------------------------------------------------------------------
# combine: permuted rows back to tokens
# --------------------------------------------------------------------------

def test_combine_reassembles_tokens(orc):
    rng = np.random.default_rng(1)
    T, k, m, E = 6, 3, 5, 7
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    counts, offsets, perm, inv = orc.dispatch(idx, E)
    vals = rng.normal(size=(T * k, m))  # value of assignment a at row inv[a]
    y_perm = np.empty_like(vals)
    y_perm[inv] = vals
    y = orc.combine(y_perm, inv, idx, w)
    for t in range(T):
        want = sum(float(w[t, j]) * vals[t * k + j] for j in np.argsort(idx[t]))
        assert np.array_equal(y[t], want)


# ---- norm of the layer's input rows (DeepSpeed-Inference summary, section 4
# fusion regions: post-attention layer norm with the intermediate GeMM) ----

def _bf16_bits(a):
    """fp32 values exactly representable in bf16 -> their bf16 bit patterns."""
    u = np.asarray(a, np.float32).view(np.uint32)
    assert np.all(u & 0xFFFF == 0)
    return (u >> 16).astype(np.uint16)


def test_norm_worked_examples(orc):
    # layer norm of [1, 2, 3, 4]: mean 2.5, biased variance 5/4, so
    # (x - 2.5) * 2 / sqrt(5) = [-3, -1, 1, 3] / sqrt(5)
    out = orc.norm(np.array([[1, 2, 3, 4]], np.float32), orc.NORM_LAYER, np.ones(4, np.float32), eps=0.0)
    assert np.allclose(out[0], np.array([-3, -1, 1, 3]) / math.sqrt(5), rtol=0, atol=1e-15)
    # RMS norm of [3, 4]: mean square 25/2, so [3, 4] * sqrt(2) / 5
    out = orc.norm(np.array([[3, 4]], np.float32), orc.NORM_RMS, np.ones(2, np.float32), eps=0.0)
    assert np.allclose(out[0], np.array([3, 4]) * math.sqrt(2) / 5, rtol=0, atol=1e-15)
    # gamma and beta per column; eps inside the square root
    g = np.array([2.0, -1.0, 0.5, 4.0], np.float32)
    b = np.array([0.25, 0.0, -1.0, 8.0], np.float32)
    out = orc.norm(np.array([[1, 2, 3, 4]], np.float32), orc.NORM_LAYER, g, b, eps=0.75)
    assert np.allclose(out[0], (np.array([-1.5, -0.5, 0.5, 1.5]) / math.sqrt(1.25 + 0.75)) * g + b, rtol=0,
                       atol=1e-14)


def test_norm_properties(orc):
    rng = np.random.default_rng(7)
    x = rng.integers(-100, 101, size=(6, 96)).astype(np.float32)
    one, zero = np.ones(96, np.float32), np.zeros(96, np.float32)
    ln = orc.norm(x, orc.NORM_LAYER, one, zero, eps=0.0)
    assert np.allclose(ln.mean(axis=1), 0.0, atol=1e-13)
    assert np.allclose((ln ** 2).mean(axis=1), 1.0, atol=1e-12)
    # invariant to a positive scale and a shift of the row (exact in fp32)
    assert np.allclose(orc.norm(2 * x + 16, orc.NORM_LAYER, one, zero, eps=0.0), ln, atol=1e-12)
    rms = orc.norm(x, orc.NORM_RMS, one, eps=0.0)
    assert np.allclose((rms ** 2).mean(axis=1), 1.0, atol=1e-12)
    assert np.allclose(orc.norm(4 * x, orc.NORM_RMS, one, eps=0.0), rms, atol=1e-12)
    # the RMS form keeps the mean: a shift changes it
    assert not np.allclose(orc.norm(x + 16, orc.NORM_RMS, one, eps=0.0), rms, atol=1e-3)
    # gamma and beta act per column on the normalised row
    g = rng.normal(size=96).astype(np.float32)
    b = rng.normal(size=96).astype(np.float32)
    assert np.allclose(orc.norm(x, orc.NORM_LAYER, g, b, eps=0.0), ln * g.astype(np.float64) + b, atol=1e-12)
    # a constant row: zero variance, so layer norm gives beta; RMS gives c / sqrt(c^2 + eps)
    c = np.full((1, 96), 3.0, np.float32)
    assert np.allclose(orc.norm(c, orc.NORM_LAYER, g, b, eps=1e-5)[0], b, atol=1e-12)
    assert np.allclose(orc.norm(c, orc.NORM_RMS, one, eps=1e-5)[0], 3.0 / math.sqrt(9.0 + 1e-5), atol=1e-15)
    # bf16 rows read as the same values
    assert np.array_equal(orc.norm(_bf16_bits(x), orc.NORM_LAYER, one, zero, eps=1e-5),
                          orc.norm(x, orc.NORM_LAYER, one, zero, eps=1e-5))


# --------------------------------------------------------------------------
# float weight formats: OCP E4M3 (fp8) and MXFP4 (E2M1 + E8M0 per 32 k)
# --------------------------------------------------------------------------

def _formats():
    with open(os.path.join(GOLDEN, "float_formats.json")) as f:
        return json.load(f)


def _num(v):
    return float("nan") if v == "nan" else float(v)


def test_fp8_decode_every_code_against_torch_and_the_definition(orc):
    """All 256 E4M3 codes (scale 1) decode as torch's float8_e4m3fn does, and
    the landmark codes of the format definition take their printed values."""
    codes = np.arange(256, dtype=np.uint8).reshape(1, 1, 256)
    ones = np.ones((1, 256), np.float32)
    got = np.array([orc.weight_value(codes, ones, "fp8", 0, 0, n) for n in range(256)])
    ref = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))
    for code, v in _formats()["e4m3_landmarks"].items():
        g = got[int(code, 16)]
        want = _num(v)
        assert (math.isnan(g) and math.isnan(want)) or (g == want and math.copysign(1, g) == math.copysign(1, want)), code
    # every finite magnitude is distinct and increasing with the code
    pos = got[:0x7F]
    assert np.all(np.diff(pos) > 0) and pos.max() == 448.0


def test_fp8_scale_is_per_output_channel(orc):
    rng = np.random.default_rng(5)
    E, K, N = 2, 6, 5
    codes = rng.integers(0, 0x7F, size=(E, K, N)).astype(np.uint8)
    codes[0, 1, 2] |= 0x80
    s = rng.random((E, N)).astype(np.float32) + 0.25
    dec = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    for e in range(E):
        for k in range(K):
            for n in range(N):
                assert orc.weight_value(codes, s, "fp8", e, k, n) == dec[e, k, n] * float(s[e, n])


def test_mxfp4_decode_every_code_and_block_scales(orc):
    """E2M1 codes decode to the MX specification's value table; the E8M0 scale
    (decoded by torch's float8_e8m0fnu) applies to the block of 32
    consecutive k of one column that holds the weight."""
    F = _formats()
    table = np.array(F["e2m1_values"])
    E, K, N = 2, 96, 4
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 16, size=(E, K, N)).astype(np.uint8)
    codes[0, :16, 0] = np.arange(16)  # every code once
    xs = rng.integers(100, 150, size=(E, K // 32, N)).astype(np.uint8)
    xs[1, 2, 3] = 127
    scale = torch.from_numpy(xs.copy()).view(torch.float8_e8m0fnu).double().numpy()
    for e in range(E):
        for k in range(K):
            for n in range(N):
                want = table[codes[e, k, n]] * scale[e, k // 32, n]
                got = orc.weight_value(codes, xs, "mxfp4", e, k, n)
                assert got == want and math.copysign(1, got) == math.copysign(1, want), (e, k, n)
    for E8, v in F["e8m0_landmarks"].items():
        dec = torch.tensor([int(E8)], dtype=torch.uint8).view(torch.float8_e8m0fnu).double().item()
        assert (math.isnan(dec) and v == "nan") or dec == _num(v), E8


@pytest.mark.parametrize("kind", ["relu", "swiglu"])
@pytest.mark.parametrize("w_dtype", ["fp8", "mxfp4"])
def test_single_float_weight_expert_is_dense_mlp(orc, syn, kind, w_dtype):
    """E = 1, k = 1 equals the torch fp64 chain on the weights dequantised
    with torch's decoders (fp8) or the MX table and torch's E8M0 decode."""
    L = _layer(syn, 9, 64, 96, 1, 1, kind, w_dtype, seed=78)
    X = orc.Experts.from_layer(L)
    r = orc.layer_forward(X, L["x"], L["wg"], None, 1)
    table = torch.tensor(_formats()["e2m1_values"], dtype=torch.float64)

    def deq(key):
        codes, s = L[key][0], L["s" + key[1:]][0]
        if w_dtype == "fp8":
            return torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double() * \
                torch.from_numpy(s.astype(np.float64))[None, :]
        sc = torch.from_numpy(s.copy()).view(torch.float8_e8m0fnu).double()
        return table[torch.from_numpy(codes.astype(np.int64))] * sc.repeat_interleave(32, dim=0)

    x = torch.from_numpy(_to64(syn, L["x"]))
    if kind == "relu":
        ref = torch.relu(x @ deq("w1")) @ deq("w2")
    else:
        ref = (torch.nn.functional.silu(x @ deq("w1")) * (x @ deq("w3"))) @ deq("w2")
    assert np.allclose(r["y"], ref.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("w_dtype", ["fp8", "fp8a8", "i8a8", "mxfp4"])
@pytest.mark.parametrize("E,k", [(3, 2), (8, 2), (8, 8)])
def test_float_weights_routed_equals_dense_masked(orc, syn, w_dtype, E, k):
    L = _layer(syn, 8, 64, 64, E, k, "swiglu", w_dtype, seed=E * 11 + k)
    X = orc.Experts.from_layer(L)
    r = orc.layer_forward(X, L["x"], L["wg"], None, k)
    assert np.array_equal(r["y"], orc.dense_masked(X, L["x"], r["idx"], r["w"]))


def test_fp8_quantisation_closed_forms(syn):
    """Per output channel s = max|W| / 448 and the largest code decodes to
    +-448; every code is within half an E4M3 step of W / s (steps 2^(e-3) for
    normals, 2^-9 below 2^-6), as torch's round-to-nearest cast of W / s."""
    E, K, N = 2, 64, 48
    q, s = syn.fp8_quant(9, syn.TID_W1, 0.02, E, K, N)
    W = syn.normal_f32(9, syn.TID_W1, 0.02, (E, K, N)).astype(np.float64)
    dec = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).double().numpy()
    assert np.allclose(s, (np.abs(W).max(axis=1) / 448).astype(np.float32), rtol=0, atol=0)
    assert np.all(np.abs(dec).max(axis=1) == 448.0)
    v = W / s[:, None, :].astype(np.float64)
    a = np.abs(v)
    step = np.where(a < 2.0**-6, 2.0**-9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0**-6))) - 3))
    assert np.all(np.abs(v - dec) <= step / 2 * (1 + 1e-12))
    cast = torch.from_numpy(v).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(dec, cast)


def test_mxfp4_quantisation_closed_forms(syn):
    """Per block of 32 k of a column: shared exponent floor(log2 max|W|) - 2
    (E8M0 = it + 127), elements the nearest E2M1 value of W / 2^X (saturated
    at 6), so within half an E2M1 step of it."""
    E, K, N = 2, 96, 24
    q, xs = syn.mxfp4_quant(9, syn.TID_W1, 0.02, E, K, N)
    W = syn.normal_f32(9, syn.TID_W1, 0.02, (E, K, N)).astype(np.float64)
    table = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    amax = np.abs(W).reshape(E, K // 32, 32, N).max(axis=2)
    X = np.floor(np.log2(amax)) - 2
    assert np.array_equal(xs.astype(np.int64), (X + 127).astype(np.int64))
    v = W / np.repeat(2.0**X, 32, axis=1)
    mag = table[q & 7]
    sign = np.where(q & 8, -1.0, 1.0)
    dec = sign * mag
    a = np.abs(v)
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    err = np.abs(v - dec)
    assert np.all((err <= step / 2 * (1 + 1e-12)) | ((a > 6) & (mag == 6)))
    assert np.all(q < 16)


# ---- fp8 activations (per-token E4M3 quantisation of the expert input) ----

def _torch_e4m3(v32):
    """Codes of torch's round-to-nearest float8_e4m3fn cast after clamping to
    the format's range (the saturating conversion)."""
    t = torch.from_numpy(np.asarray(v32, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encoder_against_torch_cast(orc):
    """Every finite bf16 value (as fp32), random fp32 values over the whole
    range, and every midpoint between neighbouring E4M3 values (the ties,
    which go to the even code) encode as torch's cast does; magnitudes from
    448 up saturate to 448."""
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    rng = np.random.default_rng(17)
    r = (rng.standard_normal(200000) * np.exp2(rng.integers(-14, 10, 200000))).astype(np.float32)
    vals = torch.from_numpy(np.arange(0, 0x7F, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (vals[1:] + vals[:-1]) / 2)  # exact in fp32
    for arr in (v, r, mids, -mids):
        assert np.array_equal(orc.e4m3_encode(arr), _torch_e4m3(arr))
    # ties: each midpoint goes to the neighbour whose mantissa is even
    got = orc.e4m3_encode(mids)
    assert np.all(got % 2 == 0)
    big = np.array([448, 450, 463.99, 464, 480, 1e30, -1e30], np.float32)
    assert np.array_equal(orc.e4m3_encode(big) & 0x7F, np.full(7, 0x7E, np.uint8))


def test_per_token_e4m3_quantisation_closed_forms(orc, syn):
    """The scale of a row is the smallest power of two s with max|x| <= 448 s
    (so max|x| / s lies in (224, 448] and nothing saturates); every code is
    torch's cast of x / s (exact in fp32); the value e4m3(code) * s is within
    half an E4M3 step (times s) of x and is a bf16 value; a row of zeros stays
    zero."""
    T, m = 40, 256
    x = syn.normal_bf16(5, syn.TID_X, 1.0, (T, m))
    x[3] = 0
    x[7] *= 0  # +0 and -0 rows alike
    x64 = _to64(syn, x)
    x64[11] *= 2.0**-20  # a small row (power-of-two scaling: exact in bf16)
    x = torch.from_numpy(x64.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(_to64(syn, x), x64)
    val, codes, scales = orc.quant_rows_e4m3(x)
    amax = np.abs(x64).max(axis=1)
    nz = amax > 0
    sc = scales.astype(np.float64)
    assert np.all(np.frexp(sc)[0] == 0.5)  # powers of two
    r = amax[nz] / sc[nz]
    assert np.all((r > 224) & (r <= 448))
    v = (x64 / sc[:, None]).astype(np.float32)
    assert np.array_equal(v.astype(np.float64), x64 / sc[:, None])  # exact scaling
    assert np.array_equal(codes, _torch_e4m3(v))
    assert np.all(val[~nz] == 0)
    dec = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(val, dec * sc[:, None])
    assert np.array_equal(torch.from_numpy(val).to(torch.bfloat16).double().numpy(), val)  # bf16 holds it
    a = np.abs(v.astype(np.float64))
    step = np.where(a < 2.0**-6, 2.0**-9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0**-6))) - 3))
    assert np.all(np.abs(v.astype(np.float64) - dec) <= step / 2 * (1 + 1e-12))


@pytest.mark.parametrize("kind", ["relu", "swiglu"])
def test_fp8a8_single_expert_is_dense_mlp_on_quantised_rows(orc, syn, kind):
    """E = 1, k = 1 with fp8 activations equals the torch fp64 chain on rows
    quantised with torch (power-of-two scale from log2 of the row maximum,
    torch's E4M3 cast) and weights dequantised with torch's decoder: the first
    projection reads the quantised row, the second the unrounded hidden row."""
    L = _layer(syn, 9, 64, 96, 1, 1, kind, "fp8a8", seed=79)
    X = orc.Experts.from_layer(L)
    r = orc.layer_forward(X, L["x"], L["wg"], None, 1)

    def deq(key):
        codes, s = L[key][0], L["s" + key[1:]][0]
        return torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double() * \
            torch.from_numpy(s.astype(np.float64))[None, :]

    x64 = _to64(syn, L["x"])
    sc = 2.0 ** np.ceil(np.log2(np.abs(x64).max(axis=1) / 448.0))
    codes = _torch_e4m3((x64 / sc[:, None]).astype(np.float32))
    xq = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double() * torch.from_numpy(sc)[:, None]
    if kind == "relu":
        ref = torch.relu(xq @ deq("w1")) @ deq("w2")
    else:
        ref = (torch.nn.functional.silu(xq @ deq("w1")) * (xq @ deq("w3"))) @ deq("w2")
    assert np.allclose(r["y"], ref.numpy(), rtol=1e-12, atol=1e-12)
    # the same weights without the activation quantisation give another result
    L8 = dict(L)
    L8["spec"] = dataclasses.replace(L["spec"], w_dtype="fp8")
    r8 = orc.layer_forward(orc.Experts.from_layer(L8), L["x"], L["wg"], None, 1)
    assert not np.allclose(r8["y"], r["y"], rtol=1e-6, atol=0)


# ---- int8 activations (per-token int8 quantisation of the expert input) ----

def test_per_token_int8_quantisation_closed_forms(orc, syn):
    """The scale of a row is the smallest power of two s with max|x| <= 127 s
    (so max|x| / s lies in (63.5, 127]); q is numpy's round-half-even of x / s
    (exact in fp64); |q| <= 127; the value q * s is a bf16 value within s / 2
    of x; a row of zeros stays zero."""
    T, m = 40, 256
    x = syn.normal_bf16(6, syn.TID_X, 1.0, (T, m))
    x[3] = 0
    x64 = _to64(syn, x)
    x64[9] *= 2.0**-25
    x64[10, :4] = [127.0, -63.5, 0.5, 1.5]  # max 127 (scale 1); ties at 0.5 and 1.5 and -63.5
    x64[10, 4:] = 0.0
    x = torch.from_numpy(x64.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(_to64(syn, x), x64)
    val, codes, scales = orc.quant_rows_i8(x)
    amax = np.abs(x64).max(axis=1)
    nz = amax > 0
    sc = scales.astype(np.float64)
    assert np.all(np.frexp(sc)[0] == 0.5)
    r = amax[nz] / sc[nz]
    assert np.all((r > 63.5) & (r <= 127))
    q = np.rint(x64 / sc[:, None])
    assert np.array_equal(codes.astype(np.float64), q)
    assert np.abs(codes.astype(np.int64)).max() <= 127
    assert np.array_equal(val, q * sc[:, None])
    assert np.all(val[~nz] == 0)
    assert np.array_equal(torch.from_numpy(val).to(torch.bfloat16).double().numpy(), val)
    assert np.all(np.abs(val - x64) <= sc[:, None] / 2)
    assert sc[10] == 1.0 and codes[10, :4].tolist() == [127, -64, 0, 2]


@pytest.mark.parametrize("kind", ["relu", "swiglu"])
def test_i8a8_single_expert_is_dense_mlp_on_quantised_rows(orc, syn, kind):
    """E = 1, k = 1 with int8 activations equals the torch fp64 chain on rows
    quantised with numpy (power-of-two scale, round half to even) and the int8
    weights times their per-channel scales."""
    L = _layer(syn, 9, 64, 96, 1, 1, kind, "i8a8", seed=80)
    X = orc.Experts.from_layer(L)
    r = orc.layer_forward(X, L["x"], L["wg"], None, 1)

    def deq(key):
        return torch.from_numpy(L[key][0].astype(np.float64) * L["s" + key[1:]][0].astype(np.float64)[None, :])

    x64 = _to64(syn, L["x"])
    sc = 2.0 ** np.ceil(np.log2(np.abs(x64).max(axis=1) / 127.0))
    xq = torch.from_numpy(np.rint(x64 / sc[:, None]) * sc[:, None])
    if kind == "relu":
        ref = torch.relu(xq @ deq("w1")) @ deq("w2")
    else:
        ref = (torch.nn.functional.silu(xq @ deq("w1")) * (xq @ deq("w3"))) @ deq("w2")
    assert np.allclose(r["y"], ref.numpy(), rtol=1e-12, atol=1e-12)
    L8 = dict(L)
    L8["spec"] = dataclasses.replace(L["spec"], w_dtype="i8")
    r8 = orc.layer_forward(orc.Experts.from_layer(L8), L["x"], L["wg"], None, 1)
    assert not np.allclose(r8["y"], r["y"], rtol=1e-6, atol=0)

