"""The layer forward captured into a HIP graph (moe_layer_graph_create) and
replayed (moe_graph_launch), against the eager forward on the same inputs
and against the CPU oracle.

Each graph is replayed several times with eager work of the program's own
(torch fills, an eager forward into another buffer) and synchronisations
between the replays, and every replay is checked; then x is rewritten in
place and a replay must follow the new input.  Paths without fp32 atomics
(decode kernels with rows and the combine kernel, the grouped GEMM) must
match the eager result bit for bit; the hybrid and fp32 paths add into an
fp32 accumulator with atomics in an arbitrary order, so there the bar is a
few fp32 roundings of the output's scale.  Every replay is also compared
with the oracle's layer (run on the GPU's router logits) at the parity bars:
bf16/int8 max|gpu - oracle| <= 2e-2 max|oracle| + 1e-3, fp32 1e-4 max|oracle|.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import mixture_experts_layer_gemv_amd as M
from mixture_experts_layer_gemv_amd.layer import MoELayer

from _gpu import assert_close, log, spec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()
    yield
    torch.cuda.synchronize()


# name, (T, m, p, E, k, kind, w_dtype, zipf), forced path ("g": grouped GEMM), bitwise
CASES = [
    ("decode_bf16", (16, 512, 1024, 8, 2, "swiglu", "bf16", None), "", True),
    ("decode_int8", (64, 512, 1024, 8, 2, "swiglu", "i8", None), "", True),
    ("skewed_split", (256, 256, 640, 16, 2, "swiglu", "bf16", 1.2), "", True),
    ("relu_bf16", (40, 256, 512, 8, 2, "relu", "bf16", None), "", True),
    ("prefill_gemm", (2048, 512, 768, 8, 2, "swiglu", "bf16", None), "g", True),
    ("tiny_f32", (32, 256, 512, 8, 2, "relu", "f32", None), "", False),
]


def _check(got, ref, bitwise, what):
    g = got.float().cpu().numpy()
    r = ref.float().cpu().numpy()
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    if bitwise:
        assert np.array_equal(g, r), f"{what}: max diff {np.abs(g - r).max()}"
    else:
        # another order of the fp32 atomic adds moves the sum by a rounding or
        # two, which a bf16 output can turn into one bf16 step
        step = 2.0**-7 if got.dtype == torch.bfloat16 else 2.0**-20
        bar = step * max(np.abs(r).max(), 1e-30)
        assert np.abs(g - r).max() <= bar, f"{what}: max diff {np.abs(g - r).max()} > {bar}"


@pytest.mark.parametrize("name,shape,path,bitwise", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(name, shape, path, bitwise, tune):
    if path:
        tune(ffn_path=M.MOE_PATH_GEMM)
    T, m, p, E, k, kind, wd, zipf = shape
    log(f"graph {name}: T={T} m={m} p={p} E={E} k={k} {kind} {wd} path={path or 'auto'}")
    L = synth.make_layer(spec(T, m, p, E, k, kind, wd, seed=T + m, zipf=zipf))
    X = oracle.Experts.from_layer(L)
    layer = MoELayer(L)

    def oracle_y(x_np):
        """The oracle's layer on x_np, routed on the GPU's logits for it."""
        dbg = layer.debug_buffers()
        layer.forward(y=layer.new_output(), dbg=dbg)
        torch.cuda.synchronize()
        ref, _, _, _ = oracle.forward_tokens(X, x_np, L["wg"], L["bias"], k, np.arange(T),
                                             logits=dbg["logits"].cpu().numpy())
        return ref

    y_eager = layer.forward().clone()
    torch.cuda.synchronize()
    ref = oracle_y(L["x"])
    g, y = layer.capture()
    try:
        other = layer.new_output()
        for rep in range(3):
            y.fill_(float("nan"))
            M.moe_graph_launch(g)
            torch.cuda.synchronize()
            _check(y, y_eager, bitwise, f"{name} replay {rep}")
            assert_close(y.float().cpu().numpy().astype(np.float64), ref, wd, f"{name} replay {rep} vs oracle")
            layer.forward(y=other)  # eager work between the replays
            other.fill_(0.0)
            torch.cuda.synchronize()
        # the graph follows the data at its pointers: new x in place
        x2 = torch.roll(layer.x, shifts=1, dims=0).contiguous()
        layer.x.copy_(x2)
        y_new = layer.forward(y=other).clone()
        ref_new = oracle_y(np.roll(L["x"], 1, axis=0))
        y.fill_(float("nan"))
        M.moe_graph_launch(g)
        torch.cuda.synchronize()
        _check(y, y_new, bitwise, f"{name} replay after new x")
        assert_close(y.float().cpu().numpy().astype(np.float64), ref_new, wd, f"{name} replay after new x vs oracle")
    finally:
        M.moe_graph_destroy(g)
        layer.close()


def test_graph_of_an_empty_batch_and_capture_refusals():
    L = synth.make_layer(spec(8, 256, 512, 8, 2, "swiglu", "bf16", seed=3))
    layer = MoELayer(L)
    y = layer.new_output()
    ws = layer.ensure_workspace(8)
    g = M.moe_layer_graph_create(layer.handle, layer.wg, layer.bias, layer.x, layer.x_dtype, 0, layer.m, layer.p,
                                 layer.E, layer.k, y, layer.y_dtype, ws, layer.ws_bytes)
    M.moe_graph_launch(g)  # no launches recorded: a no-op
    torch.cuda.synchronize()
    M.moe_graph_destroy(g)
    # a bad argument fails the capture with the forward's own error
    with pytest.raises(M.MoeError) as ei:
        M.moe_layer_graph_create(layer.handle, layer.wg, layer.bias, layer.x, layer.x_dtype, 8, layer.m + 1, layer.p,
                                 layer.E, layer.k, y, layer.y_dtype, ws, layer.ws_bytes)
    assert ei.value.status == M.MOE_ERR_INVALID_ARG
    # refused while the profiler brackets launches with events
    M.moe_profile_begin(16)
    try:
        with pytest.raises(M.MoeError) as ei:
            layer.capture()
        assert ei.value.status == M.MOE_ERR_INVALID_ARG
    finally:
        M.moe_profile_end()
    # and works again afterwards
    g, y = layer.capture()
    M.moe_graph_launch(g)
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()
    M.moe_graph_destroy(g)
    layer.close()
