"""fp8 (OCP E4M3 with per-output-channel scales) and MXFP4 (E2M1 with one
E8M0 scale per 32 k) weights on the decode kernels, against the CPU oracle.

The kernels convert the weights exactly to bf16 in registers (the hardware
conversions; MXFP4 with its block scale applied in the same instruction) and
multiply on the bf16 matrix cores with fp32 accumulation, so the bar is the
bf16 one: max|gpu - oracle| <= 2e-2 max|oracle| + 1e-3.  Cases: the expert
stage on explicit dispatches and the whole layer, over ragged and empty
experts, both expert kinds, every decode launch form (one or two M tiles,
gathered or packed rows, reduction or columns split over the waves), and the
Mixtral-shaped decode layers at full size on every token.
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


@pytest.mark.parametrize("w_dtype", ["fp8", "mxfp4"])
@pytest.mark.parametrize("kind", ["swiglu", "relu"])
@pytest.mark.parametrize("T,m,p,E,k", SHAPES)
def test_float_weights_expert_stage_and_layer(w_dtype, kind, T, m, p, E, k):
    log(f"{w_dtype} kind={kind} T={T} m={m} p={p} E={E} k={k}")
    L = synth.make_layer(spec(T, m, p, E, k, kind, w_dtype, seed=T + p + 3, sw=0.05, sr=0.05))
    layer = MoELayer(L)
    rng = np.random.default_rng(T)
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


@pytest.mark.parametrize("w_dtype", ["fp8", "mxfp4"])
@pytest.mark.parametrize("mt", [1, 2])
@pytest.mark.parametrize("pack", [0, 1])
@pytest.mark.parametrize("waves", ["k", "n"])
def test_float_weights_launch_modes(w_dtype, mt, pack, waves, tune):
    tune(ffn_path=M.MOE_PATH_SKINNY, skinny_mt=mt, skinny_pack=1 if pack else -1,
         skinny_splitk=1 if waves == "k" else -1)
    log(f"{w_dtype} modes mt={mt} pack={pack} waves={waves}")
    _layer_check(synth.make_layer(spec(61, 256, 384, 8, 2, "swiglu", w_dtype, seed=mt + 2 * pack, zipf=1.2,
                                       sw=0.05, sr=0.05)))


MX_GEMM_SHAPES = [(5, 128, 128, 3, 2), (37, 256, 384, 8, 2), (300, 256, 512, 4, 2), (600, 1024, 1536, 8, 2),
                  (1, 512, 384, 16, 2), (64, 128, 128, 64, 4), (700, 384, 256, 2, 1)]


@pytest.mark.parametrize("kind", ["swiglu", "relu"])
@pytest.mark.parametrize("T,m,p,E,k", MX_GEMM_SHAPES)
def test_mxfp4_grouped_gemm(kind, T, m, p, E, k, tune):
    """MXFP4 weights on the grouped GEMM (forced onto small shapes): each
    projection's weights expanded to packed bf16 in the workspace, then the
    bf16 kernel; the expert stage on an explicit dispatch (ragged and empty
    experts) and the whole layer."""
    tune(ffn_path=M.MOE_PATH_GEMM)
    log(f"mxfp4 gemm kind={kind} T={T} m={m} p={p} E={E} k={k}")
    L = synth.make_layer(spec(T, m, p, E, k, kind, "mxfp4", seed=T + 5 * E + p, sw=0.05, sr=0.05))
    layer = MoELayer(L)
    rng = np.random.default_rng(T + 3)
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


@pytest.mark.parametrize("cfg", ["c9", "c10"])
def test_float_weight_decode_layers_full_size(cfg):
    sp = synth.spec(cfg)
    log(f"{sp.name}, full size, every token")
    _layer_check(synth.make_layer(sp))


def test_float_weights_refuse_unsupported_shapes():
    L = synth.make_layer(spec(4, 192, 256, 4, 1, "swiglu", "mxfp4", seed=1))
    with pytest.raises(M.MoeError) as ei:
        MoELayer(L)
    assert ei.value.status == M.MOE_ERR_UNSUPPORTED
