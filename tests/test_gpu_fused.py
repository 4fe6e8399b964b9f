"""moe_layer_forward_fused: the layer's input norm done in the routing pass
and the residual added at the end (DeepSpeed-Inference summary, section 4
fusion regions), against the oracle.

The normalised rows the GPU returns (x_norm) must lie within one step of
the activation dtype (plus fp32 reduction error) of the oracle's norm of x.
The rest of the layer is then checked from those rows: the oracle's logits
of x_norm against the GPU's within the fp32 bound, the top-k bit for bit on
the GPU's logits, and y against the oracle layer on x_norm plus the residual
at the usual bars, on every expert path.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import mixture_experts_layer_gemv_amd as M
from mixture_experts_layer_gemv_amd.layer import MoELayer, to_device

from _gpu import assert_close, log, logit_bound, spec, y_to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()
    yield
    torch.cuda.synchronize()


# name, (T, m, p, E, k, kind, w_dtype, zipf), forced path ("g": grouped GEMM)
PATHS = [
    ("decode_bf16", (16, 512, 1024, 8, 2, "swiglu", "bf16", None), ""),
    ("decode_int8", (64, 512, 1024, 8, 2, "swiglu", "i8", None), ""),
    ("skewed_split", (256, 256, 640, 16, 2, "swiglu", "bf16", 1.2), ""),
    ("relu_e12", (40, 256, 512, 12, 3, "relu", "bf16", None), ""),  # E=12: the unfused norm kernel
    # past 1024 tokens the staged router takes eight tokens per block: a
    # ragged last block of four
    ("prefill_gemm", (2052, 512, 768, 8, 2, "swiglu", "bf16", None), "g"),
    ("tiny_f32", (32, 256, 512, 8, 2, "relu", "f32", None), ""),
    # 8-bit activations: the normalised rows quantised in the routing pass
    # (E = 8), or by the quantisation kernel after the norm kernel (E = 12)
    ("decode_fp8a8", (64, 512, 1024, 8, 2, "swiglu", "fp8a8", None), ""),
    ("prefill_i8a8", (1100, 512, 768, 8, 2, "swiglu", "i8a8", None), "g"),
    ("relu_e12_fp8a8", (40, 256, 512, 12, 3, "relu", "fp8a8", None), ""),
]
FUSIONS = [("layer", True), ("rms", False), ("none", True)]
NORM = {"none": M.MOE_NORM_NONE, "layer": M.MOE_NORM_LAYER, "rms": M.MOE_NORM_RMS}
ONORM = {"layer": oracle.NORM_LAYER, "rms": oracle.NORM_RMS}


def _x64(a):
    return synth.bf16_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


@pytest.mark.parametrize("norm,with_res", FUSIONS, ids=[f"{n}{'_res' if r else ''}" for n, r in FUSIONS])
@pytest.mark.parametrize("name,shape,path", PATHS, ids=[c[0] for c in PATHS])
def test_fused_forward(name, shape, path, norm, with_res, tune):
    if path:
        tune(ffn_path=M.MOE_PATH_GEMM)
    T, m, p, E, k, kind, wd, zipf = shape
    log(f"fused {name} norm={norm} residual={with_res}: T={T} m={m} p={p} E={E} k={k} {kind} {wd}")
    L = synth.make_layer(spec(T, m, p, E, k, kind, wd, seed=T + 7 * m, zipf=zipf))
    rng = np.random.default_rng(T + m)
    gamma = (1.0 + 0.1 * rng.standard_normal(m)).astype(np.float32)
    beta = (0.05 * rng.standard_normal(m)).astype(np.float32) if norm == "layer" else None
    eps = 1e-5
    layer = MoELayer(L)
    y = layer.new_output()
    ydt = y.dtype
    res = (0.5 * torch.randn(T, m, generator=torch.Generator().manual_seed(T), dtype=torch.float32)).to(ydt)
    res = res.to("cuda") if with_res else None
    xn = torch.empty_like(layer.x) if norm != "none" else None
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    tw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ws = layer.ensure_workspace(T)
    M.moe_layer_forward_fused(layer.handle, layer.wg, layer.bias, layer.x, layer.x_dtype, NORM[norm],
                              to_device(gamma) if norm != "none" else None,
                              to_device(beta) if beta is not None else None, eps, res, T, m, p, E, k, y,
                              layer.y_dtype, ws, layer.ws_bytes, xn, idx, tw, lg)
    torch.cuda.synchronize()
    # 1. the normalised rows
    if norm != "none":
        ref_n = oracle.norm(L["x"], ONORM[norm], gamma, beta, eps)
        got_n = xn.float().cpu().numpy().astype(np.float64) if xn.dtype == torch.bfloat16 else \
            xn.cpu().numpy().astype(np.float64)
        step = 2.0**-7 if xn.dtype == torch.bfloat16 else 2.0**-22
        bar = (step + 1e-4) * np.abs(ref_n) + 1e-4 * (np.abs(beta)[None, :] if beta is not None else 0.0) + 1e-6
        err = np.abs(got_n - ref_n)
        log(f"  x_norm: max|err|={err.max():.3e}, worst err/bar={np.max(err / bar):.3f}")
        assert np.all(err <= bar), "normalised rows outside one step of the oracle's norm"
        xn_np = xn.view(torch.int16).cpu().numpy().view(np.uint16) if xn.dtype == torch.bfloat16 else \
            xn.cpu().numpy()
    else:
        xn_np = L["x"]
    # 2. routing on the normalised rows
    lg_g = lg.cpu().numpy()
    ref_lg = oracle.router_logits(xn_np, L["wg"], L["bias"])
    assert np.all(np.abs(lg_g.astype(np.float64) - ref_lg) <= logit_bound(_x64(xn_np), L["wg"], L["bias"]))
    idx_o, _ = oracle.topk(lg_g, k)
    assert np.array_equal(idx.cpu().numpy(), idx_o)
    # 3. the layer on the normalised rows, plus the residual
    ref, i_o, _, _ = oracle.forward_tokens(oracle.Experts.from_layer(L), xn_np, L["wg"], L["bias"], k,
                                           np.arange(T), logits=lg_g)
    assert np.array_equal(i_o, idx.cpu().numpy())
    if with_res:
        ref = ref + res.float().cpu().numpy().astype(np.float64)
    assert_close(y_to_np(y), ref, wd, "y")
    layer.close()


def test_fused_argument_errors():
    L = synth.make_layer(spec(8, 256, 512, 8, 2, "swiglu", "bf16", seed=1))
    layer = MoELayer(L)
    y = layer.new_output()
    ws = layer.ensure_workspace(8)
    g = to_device(np.ones(256, np.float32))
    g_mis = to_device(np.ones(257, np.float32))[1:]  # 4 bytes past a 16-byte boundary
    args = lambda norm, gamma, beta, eps: (layer.handle, layer.wg, layer.bias, layer.x, layer.x_dtype, norm, gamma,
                                           beta, eps, None, 8, 256, 512, 8, 2, y, layer.y_dtype, ws, layer.ws_bytes)
    for bad in [(7, g, None, 1e-5), (M.MOE_NORM_LAYER, None, None, 1e-5), (M.MOE_NORM_RMS, g, g, 1e-5),
                (M.MOE_NORM_NONE, g, None, 1e-5), (M.MOE_NORM_LAYER, g, None, -1.0),
                (M.MOE_NORM_LAYER, g, None, float("nan")), (M.MOE_NORM_LAYER, g_mis, None, 1e-5),
                (M.MOE_NORM_LAYER, g, g_mis, 1e-5)]:
        with pytest.raises(M.MoeError) as ei:
            M.moe_layer_forward_fused(*args(*bad))
        assert ei.value.status == M.MOE_ERR_INVALID_ARG, bad
    # no fusion: the same bits as moe_layer_forward
    y0 = layer.forward().clone()
    M.moe_layer_forward_fused(*args(M.MOE_NORM_NONE, None, None, 0.0))
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    layer.close()
