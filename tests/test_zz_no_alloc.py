"""The allocation-free forward (moe_layer_forward_noalloc) against the
forward with a caller workspace (moe_layer_forward).

Both run the same kernels on the same inputs; only the workspace differs (a
static device array of the library against a torch allocation), so on paths
without atomics the outputs must agree bit for bit, and every path stays at
the oracle's parity bar.  Two calls in a row on the same GPU, the second with
a smaller batch, check that nothing the first left in the shared array leaks
into the second.  A batch whose workspace exceeds the array is refused before
anything is launched.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import mixture_experts_layer_gemv_amd as M
from mixture_experts_layer_gemv_amd.layer import MoELayer, to_device

from _gpu import assert_close, log, spec, y_to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()
    yield
    torch.cuda.synchronize()


def _noalloc(layer, x, T):
    y = layer.new_output(T)
    y.fill_(float("nan"))
    M.moe_layer_forward_noalloc(layer.handle, layer.wg, layer.bias, x, layer.x_dtype, T, layer.m, layer.p, layer.E,
                                layer.k, y, layer.y_dtype)
    return y


def _reference(layer, x, T):
    y = layer.new_output(T)
    layer.forward(x=x, y=y, T=T)
    return y


# name, (T, m, p, E, k, kind, w_dtype, zipf), second T, bitwise
CASES = [
    ("decode_bf16", (48, 512, 1024, 8, 2, "swiglu", "bf16", None), 16, True),
    ("decode_int8", (64, 512, 1024, 8, 2, "swiglu", "i8", None), 5, True),
    ("decode_int4", (40, 256, 512, 8, 2, "swiglu", "i4", None), 7, True),
    ("skewed_split", (256, 256, 640, 16, 2, "swiglu", "bf16", 1.2), 100, True),
    ("relu_bf16", (40, 256, 512, 8, 2, "relu", "bf16", None), 3, True),
    ("prefill_gemm", (1536, 256, 512, 4, 2, "swiglu", "bf16", None), 600, True),
    ("tiny_f32", (32, 256, 512, 8, 2, "relu", "f32", None), 9, False),
    # the routing pass's 8-bit quantised rows, and MXFP4 weights expanded to
    # bf16, in the scratch too
    ("decode_fp8a8", (64, 256, 512, 8, 2, "swiglu", "fp8a8", None), 9, True),
    ("prefill_gemm_i8a8", (1536, 256, 512, 4, 2, "swiglu", "i8a8", None), 600, True),
    ("prefill_gemm_mxfp4", (1536, 256, 512, 4, 2, "swiglu", "mxfp4", None), 600, True),
]


@pytest.mark.parametrize("name,shape,t2,bitwise", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_forward(name, shape, t2, bitwise):
    T, m, p, E, k, kind, wd, zipf = shape
    log(f"noalloc {name}: T={T} then {t2}, m={m} p={p} E={E} k={k} {kind} {wd}")
    L = synth.make_layer(spec(T, m, p, E, k, kind, wd, seed=T + p, zipf=zipf, sw=0.05, sr=0.05))
    X = oracle.Experts.from_layer(L)
    layer = MoELayer(L)
    for Tc in (T, t2):  # two calls in a row, the second smaller
        x = layer.x[:Tc].contiguous()
        y_na = _noalloc(layer, x, Tc)
        y_ws = _reference(layer, x, Tc)
        torch.cuda.synchronize()
        got, want = y_to_np(y_na), y_to_np(y_ws)
        assert np.all(np.isfinite(got)), f"{name} T={Tc}: rows left unwritten"
        if bitwise:
            assert np.array_equal(got, want), f"{name} T={Tc}: max diff {np.abs(got - want).max()}"
        # the oracle's layer on the GPU's logits for these tokens
        dbg = layer.debug_buffers(Tc)
        layer.forward(x=x, y=layer.new_output(Tc), T=Tc, dbg=dbg)
        torch.cuda.synchronize()
        x_np = L["x"][:Tc]
        ref, _, _, _ = oracle.forward_tokens(X, x_np, L["wg"], L["bias"], k, np.arange(Tc),
                                             logits=dbg["logits"].cpu().numpy())
        assert_close(got, ref, wd, f"{name} T={Tc} noalloc vs oracle")
    layer.close()


def test_noalloc_refuses_a_batch_beyond_its_scratch():
    T, m, p, E, k = 4096, 1024, 2048, 8, 2
    need = M.moe_workspace_size_for(m, p, E, M.MOE_SWIGLU, M.MOE_BF16, None, T, k)
    assert need > M.MOE_NOALLOC_SCRATCH_BYTES
    L = synth.make_layer(spec(8, m, p, E, k, "swiglu", "bf16", seed=2))
    layer = MoELayer(L)
    x = torch.zeros((T, m), dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, m), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(M.MoeError) as ei:
        M.moe_layer_forward_noalloc(layer.handle, layer.wg, layer.bias, x, layer.x_dtype, T, m, p, E, k, y,
                                    layer.y_dtype)
    assert ei.value.status == M.MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((y.float() == 7.0).all()), "a refused call must launch nothing"
    # T = 0 is a no-op, and a small batch still runs after the refusal
    M.moe_layer_forward_noalloc(layer.handle, layer.wg, layer.bias, x, layer.x_dtype, 0, m, p, E, k, y, layer.y_dtype)
    y8 = _noalloc(layer, layer.x, 8)
    torch.cuda.synchronize()
    assert np.array_equal(y_to_np(y8), y_to_np(_reference(layer, layer.x, 8)))
    layer.close()
