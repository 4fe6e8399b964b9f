"""8-bit activations (MOE_FP8A8 and MOE_I8A8 layers) against the CPU oracle.

Each token's input to the experts is quantised to E4M3 (or int8) with one
power-of-two scale per token; the quantised values are bf16 values, so the
layer's numbers are those of the oracle's fp8a8 (i8a8) expert on every path,
and at prefill sizes the first projection multiplies the codes on the fp8
(int8) matrix cores.  Checked: the quantisation step alone, bit for bit
(codes are decided by floating point on both sides in the same exact
arithmetic: a division by a power of two and a round-to-nearest-even), then
the expert stage and the whole layer at the bf16 bar over expert kinds,
ragged and empty experts, every decode launch form and the grouped GEMM
forced onto small shapes.
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


def _bf16_bits(a64):
    return torch.from_numpy(np.asarray(a64, np.float64)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rows_under_test(T, m, seed):
    """bf16 rows over many magnitudes, with zero rows, negative zeros, rows
    whose maximum sits exactly on 448 * 2^X and on the next bf16 value above
    it, and entries on the E4M3 rounding ties of their row's scale."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, m)) * np.exp2(rng.integers(-30, 30, size=(T, 1)))
    x[0] = 0.0
    x[1] = -0.0
    x[2, ::3] = -0.0
    x[3] = np.linspace(-1, 1, m) * 448.0  # max exactly 448: scale 1
    x[4] = x[3] * (1 + 2.0**-7)  # max just above 448 * 2^0: scale 2
    ties = torch.from_numpy(np.arange(0, 0x7E, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    mids = (ties[1:] + ties[:-1]) / 2  # exact in bf16 for the small exponents used here
    for r in (5, 6):
        row = np.zeros(m)
        row[0] = 448.0  # scale 1 (r = 5) and 2^-4 (r = 6)
        row[1:1 + len(mids)] = mids[: m - 1]
        x[r] = row * (1.0 if r == 5 else 2.0**-4)
    xb = _bf16_bits(x)
    return xb


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
@pytest.mark.parametrize("T,m", [(8, 64), (40, 256), (300, 4096)])
def test_quantize_rows_is_bit_exact(fmt, T, m):
    xb = _rows_under_test(T, m, seed=T + m)
    if fmt == "i8":  # rows whose maximum sits on 127 * 2^X, and the int8 ties
        x64 = torch.from_numpy(xb.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
        x64[5, :8] = [127, 0.5, 1.5, -2.5, 126.5, -63.5, 3.5, 100]
        x64[6] = x64[5] * 2.0**-9
        xb = _bf16_bits(x64)
    val, codes, scales = (oracle.quant_rows_i8 if fmt == "i8" else oracle.quant_rows_e4m3)(xb)
    x = to_device(xb)
    xq = torch.empty((T, m), dtype=torch.int16, device="cuda")
    sc = torch.empty(T, dtype=torch.float32, device="cuda")
    (M.moe_quantize_rows_i8 if fmt == "i8" else M.moe_quantize_rows_e4m3)(x, T, m, xq, sc)
    torch.cuda.synchronize()
    got_s = sc.cpu().numpy()
    assert np.array_equal(got_s, scales), "scales"
    got = xq.cpu().numpy().view(np.uint16)
    want = _bf16_bits(val)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} values differ, first at {bad[:5].tolist()}"


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
def test_quantize_rows_every_bf16_value(fmt):
    """Every bf16 value of magnitude up to the format's largest (448 for
    E4M3, 127 for int8), both signs, in rows whose maximum is exactly that
    bound, so the scale is 1 and each value's code is the format's rounding
    of the value itself: the kernel's codes (as their values) against the
    oracle's for the whole input range of the encoder."""
    qmax = 448.0 if fmt == "e4m3" else 127.0
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    keep = np.isfinite(v) & (np.abs(v) <= qmax)
    vals = bits[keep]
    m = 4096
    per = m - 1
    T = (len(vals) + per - 1) // per
    xb = np.zeros((T, m), np.uint16)
    top = _bf16_bits(np.array([qmax]))[0]
    xb[:, 0] = top
    flat = np.zeros(T * per, np.uint16)
    flat[: len(vals)] = vals
    xb[:, 1:] = flat.reshape(T, per)
    val, codes, scales = (oracle.quant_rows_i8 if fmt == "i8" else oracle.quant_rows_e4m3)(xb)
    assert np.all(scales == 1.0)
    x = to_device(xb)
    xq = torch.empty((T, m), dtype=torch.int16, device="cuda")
    sc = torch.empty(T, dtype=torch.float32, device="cuda")
    (M.moe_quantize_rows_i8 if fmt == "i8" else M.moe_quantize_rows_e4m3)(x, T, m, xq, sc)
    torch.cuda.synchronize()
    assert np.all(sc.cpu().numpy() == 1.0), "scales"
    got = xq.cpu().numpy().view(np.uint16)
    want = _bf16_bits(val)
    bad = np.argwhere(got != want)
    log(f"{fmt}: {len(vals)} bf16 values over {T} rows, {len(bad)} differ")
    assert bad.size == 0, f"{len(bad)} values differ, first inputs {[hex(xb[i, j]) for i, j in bad[:5]]}"


SHAPES = [(1, 128, 256, 4, 1), (16, 512, 1024, 8, 2), (64, 256, 384, 8, 2), (257, 256, 512, 16, 2),
          (3, 128, 128, 8, 8)]


def _layer_check(L):
    sp = L["spec"]
    layer = MoELayer(L)
    dbg = layer.debug_buffers()
    y = layer.forward(dbg=dbg)
    torch.cuda.synchronize()
    lg, idx_g, _, counts, _ = check_routing(L, dbg, sp.T, sp.E, sp.k)
    log(f"  counts={counts.tolist()}")
    ref, i_o, _, _ = oracle.forward_tokens(oracle.Experts.from_layer(L), L["x"], L["wg"], L["bias"], sp.k,
                                           np.arange(sp.T), logits=lg)
    assert np.array_equal(i_o, idx_g)
    assert_close(y_to_np(y), ref, "bf16", f"y[{sp.T} tokens]")
    layer.close()


@pytest.mark.parametrize("wd", ["fp8a8", "i8a8"])
@pytest.mark.parametrize("kind", ["swiglu", "relu"])
@pytest.mark.parametrize("T,m,p,E,k", SHAPES)
def test_act8_expert_stage_and_layer(wd, kind, T, m, p, E, k):
    log(f"{wd} kind={kind} T={T} m={m} p={p} E={E} k={k}")
    L = synth.make_layer(spec(T, m, p, E, k, kind, wd, seed=T + p + 4, sw=0.05, sr=0.05))
    layer = MoELayer(L)
    rng = np.random.default_rng(T + 1)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, _ = oracle.dispatch(idx, E)
    y_perm = torch.full((T * k, m), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(layer.handle, layer.x, layer.x_dtype, T, m, p, E, k, to_device(perm), to_device(offsets),
                     y_perm, layer.ensure_workspace(T), layer.ws_bytes)
    torch.cuda.synchronize()
    ref, _ = oracle.expert_rows(oracle.Experts.from_layer(L), L["x"], k, perm, offsets)
    got = y_perm.cpu().numpy()
    assert np.all(np.isfinite(got)), "rows left unwritten"
    assert_close(got, ref, "bf16", "y_perm")
    layer.close()
    _layer_check(L)


@pytest.mark.parametrize("wd", ["fp8a8", "i8a8"])
@pytest.mark.parametrize("mt", [1, 2])
@pytest.mark.parametrize("pack", [0, 1])
@pytest.mark.parametrize("waves", ["k", "n"])
def test_act8_decode_launch_modes(wd, mt, pack, waves, tune):
    tune(ffn_path=M.MOE_PATH_SKINNY, skinny_mt=mt, skinny_pack=1 if pack else -1,
         skinny_splitk=1 if waves == "k" else -1)
    log(f"{wd} modes mt={mt} pack={pack} waves={waves}")
    _layer_check(synth.make_layer(spec(61, 256, 384, 8, 2, "swiglu", wd, seed=mt + 2 * pack + 1, zipf=1.2,
                                       sw=0.05, sr=0.05)))


GEMM_SHAPES = [(5, 64, 128, 3, 2), (37, 192, 320, 8, 2), (300, 256, 512, 4, 2), (600, 1024, 1536, 8, 2),
               (1, 512, 384, 16, 2), (64, 128, 128, 64, 4), (700, 320, 192, 2, 1)]


@pytest.mark.parametrize("wd", ["fp8a8", "i8a8"])
@pytest.mark.parametrize("kind", ["swiglu", "relu"])
@pytest.mark.parametrize("T,m,p,E,k", GEMM_SHAPES)
def test_act8_grouped_gemm(wd, kind, T, m, p, E, k, tune):
    tune(ffn_path=M.MOE_PATH_GEMM)
    log(f"{wd} gemm kind={kind} T={T} m={m} p={p} E={E} k={k}")
    L = synth.make_layer(spec(T, m, p, E, k, kind, wd, seed=T + 3 * E + p, sw=0.05, sr=0.05))
    layer = MoELayer(L)
    rng = np.random.default_rng(T + 2)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, _ = oracle.dispatch(idx, E)
    y_perm = torch.full((T * k, m), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(layer.handle, layer.x, layer.x_dtype, T, m, p, E, k, to_device(perm), to_device(offsets),
                     y_perm, layer.ensure_workspace(T), layer.ws_bytes)
    torch.cuda.synchronize()
    ref, _ = oracle.expert_rows(oracle.Experts.from_layer(L), L["x"], k, perm, offsets)
    got = y_perm.cpu().numpy()
    assert np.all(np.isfinite(got)), "rows left unwritten"
    assert_close(got, ref, "bf16", "y_perm")
    layer.close()
    _layer_check(L)


@pytest.mark.parametrize("wd", ["fp8a8", "i8a8"])
@pytest.mark.parametrize("path", ["skinny", "gemm"])
@pytest.mark.parametrize("T,m,p,E,k", [(40, 256, 384, 8, 2), (300, 512, 256, 16, 2), (3, 128, 128, 64, 4),
                                       # past 1024 tokens: eight tokens per routing block, a ragged last one
                                       (1100, 256, 256, 8, 2), (1030, 512, 256, 16, 2)])
def test_act8_quantised_in_routing_pass(wd, path, T, m, p, E, k, tune):
    """The layer quantises its experts' input rows inside the routing pass
    (route_quant on, the default); the same layer with the quantisation
    kernel instead (off) must give the same output bits, and both the
    oracle's numbers."""
    log(f"{wd} {path} route_quant on/off T={T} m={m} p={p} E={E} k={k}")
    L = synth.make_layer(spec(T, m, p, E, k, "swiglu", wd, seed=T + E, sw=0.05, sr=0.05))
    outs = []
    for rq in (1, -1):
        tune(ffn_path=M.MOE_PATH_GEMM if path == "gemm" else M.MOE_PATH_SKINNY, route_quant=rq)
        layer = MoELayer(L)
        y = layer.forward()
        torch.cuda.synchronize()
        outs.append(y.clone())
        layer.close()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), "route_quant on/off differ"
    tune(route_quant=0)
    _layer_check(L)


def test_fp8a8_decode_layer_full_size():
    sp = synth.spec("c13")
    log(f"{sp.name}, full size, every token")
    _layer_check(synth.make_layer(sp))
