"""int4 weights (W4A16: q in [-7, 7] held two per byte, per-output-channel
fp32 scales, bf16 activations), a next row after the int8 layer, against the
oracle's q * s experts.

The expert stage and the whole layer over ragged, empty-expert and skewed
shapes (m and p multiples of 128), every launch mode of the decode kernels
(M tiles, packed or gathered rows, waves splitting columns or the
reduction), the unsupported shapes, and the full-size int4 decode layer on
sampled tokens.  Bars as for bf16 and int8 weights.
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


def _layer_check(L, sample=None):
    sp = L["spec"]
    layer = MoELayer(L)
    dbg = layer.debug_buffers()
    y = layer.forward(dbg=dbg)
    torch.cuda.synchronize()
    lg, idx_g, _, counts, _ = check_routing(L, dbg, sp.T, sp.E, sp.k)
    log(f"  counts={counts.tolist()}")
    tokens = np.arange(sp.T) if sample is None else np.sort(
        np.random.default_rng(1).choice(sp.T, size=min(sample, sp.T), replace=False))
    ref, i_o, _, _ = oracle.forward_tokens(oracle.Experts.from_layer(L), L["x"], L["wg"], L["bias"], sp.k, tokens,
                                           logits=lg)
    assert np.array_equal(i_o, idx_g[tokens])
    assert_close(y_to_np(y)[tokens], ref, "i4", f"y[{len(tokens)} tokens]")
    layer.close()


@pytest.mark.parametrize("kind", ["swiglu", "relu"])
@pytest.mark.parametrize("T,m,p,E,k", SHAPES)
def test_int4_expert_stage_and_layer(kind, T, m, p, E, k):
    log(f"int4 kind={kind} T={T} m={m} p={p} E={E} k={k}")
    L = synth.make_layer(spec(T, m, p, E, k, kind, "i4", seed=T + p, sw=0.05, sr=0.05))
    layer = MoELayer(L)
    rng = np.random.default_rng(T)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, _ = oracle.dispatch(idx, E)
    y_perm = torch.empty((T * k, m), dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(layer.handle, layer.x, layer.x_dtype, T, m, p, E, k, to_device(perm), to_device(offsets),
                     y_perm, layer.ensure_workspace(T), layer.ws_bytes)
    torch.cuda.synchronize()
    ref, _ = oracle.expert_rows(oracle.Experts.from_layer(L), L["x"], k, perm, offsets)
    assert_close(y_perm.cpu().numpy(), ref, "i4", "y_perm")
    layer.close()
    _layer_check(L)


@pytest.mark.parametrize("mt", [1, 2])
@pytest.mark.parametrize("pack", [0, 1])
@pytest.mark.parametrize("waves", ["k", "n"])
def test_int4_launch_modes(mt, pack, waves, tune):
    tune(ffn_path=M.MOE_PATH_SKINNY, skinny_mt=mt, skinny_pack=1 if pack else -1,
         skinny_splitk=1 if waves == "k" else -1)
    log(f"int4 modes mt={mt} pack={pack} waves={waves}")
    _layer_check(synth.make_layer(spec(61, 256, 384, 8, 2, "swiglu", "i4", seed=mt + 2 * pack, zipf=1.2, sw=0.05,
                                       sr=0.05)))


def test_int4_needs_multiples_of_128():
    L = synth.make_layer(spec(4, 192, 256, 4, 1, "swiglu", "i4", seed=1))
    with pytest.raises(M.MoeError) as ei:
        MoELayer(L)
    assert ei.value.status == M.MOE_ERR_UNSUPPORTED


def test_int4_decode_layer_full_size():
    log("int4 decode layer, full size, every token")
    _layer_check(synth.make_layer(synth.spec("c6")))


def test_int4_relu_layer_long_reduction():
    """ReLU experts at the Mixtral shape: the down projection reduces over
    p = 14336 nonnegative activations, where removing the int4 storage offset
    (136 * sum x, subtracted after the fp32 accumulation) cancels the most;
    every token is checked at the bf16 bar."""
    log("int4 ReLU layer, m=4096 p=14336, every token")
    _layer_check(synth.make_layer(spec(64, 4096, 14336, 8, 2, "relu", "i4", seed=6)))
