"""The decode FFN's launch variants against the CPU oracle.

The skinny kernels run with 1, 2 or 4 M tiles of 16 rows per work item,
read their activations either gathered row by row or as packed 1 KiB
fragments (x packed by k_pack_rows, H written packed by the up projection),
and split a work item over their four waves either along the reduction
(partials summed through LDS) or along the columns.  The library picks these
from the mean rows per expert; here every combination is forced
(moe_tuning's skinny_mt, skinny_pack, skinny_splitk) on bf16 and int8 layers
with ragged experts, for the layer and the expert-FFN stage, at the bars of
the other parity tests; so are the activation sharing through LDS
(skinny_shared), the down projection's epilogue (unweighted rows and the
combine kernel, or weighted atomics: down_rows) and its reduction slices.
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


@pytest.mark.parametrize("w_dtype", ["bf16", "i8"])
@pytest.mark.parametrize("mt", [1, 2, 4])
@pytest.mark.parametrize("pack", [0, 1])
@pytest.mark.parametrize("waves", ["k", "n"])
@pytest.mark.parametrize("T,m,p,E,k,zipf", [(61, 256, 320, 8, 2, 1.2), (100, 192, 256, 4, 1, None)])
def test_skinny_mode_layer(w_dtype, mt, pack, waves, T, m, p, E, k, zipf, tune):
    tune(ffn_path=M.MOE_PATH_SKINNY, skinny_mt=mt, skinny_pack=1 if pack else -1,
         skinny_splitk=1 if waves == "k" else -1)
    log(f"skinny layer w={w_dtype} mt={mt} pack={pack} waves={waves} T={T} m={m} p={p} E={E} k={k}")
    L = synth.make_layer(spec(T, m, p, E, k, "swiglu", w_dtype, seed=T + mt + 7 * pack, zipf=zipf, sw=0.05,
                              sr=0.05))
    layer = MoELayer(L)
    dbg = layer.debug_buffers()
    y = layer.forward(dbg=dbg)
    torch.cuda.synchronize()
    lg, idx_g, _, counts, _ = check_routing(L, dbg, T, E, k)
    log(f"  counts={counts.tolist()}")
    ref, i_o, _, _ = oracle.forward_tokens(oracle.Experts.from_layer(L), L["x"], L["wg"], L["bias"], k,
                                           np.arange(T), logits=lg)
    assert np.array_equal(i_o, idx_g)
    assert_close(y_to_np(y), ref, w_dtype, "y")
    layer.close()


@pytest.mark.parametrize("kind", ["swiglu", "relu"])
@pytest.mark.parametrize("mt", [2, 4])
@pytest.mark.parametrize("waves", ["k", "n"])
def test_skinny_packed_expert_ffn_stage(kind, mt, waves, tune):
    tune(ffn_path=M.MOE_PATH_SKINNY, skinny_mt=mt, skinny_pack=1, skinny_splitk=1 if waves == "k" else -1)
    T, m, p, E, k = 90, 128, 384, 6, 2
    L = synth.make_layer(spec(T, m, p, E, k, kind, "bf16", seed=31 + mt, sw=0.05))
    layer = MoELayer(L)
    rng = np.random.default_rng(mt)
    # the first 40 tokens all pick expert 2, so it holds well over one chunk
    idx = np.stack([np.concatenate([[2], rng.permutation([e for e in range(E) if e != 2])[:k - 1]]) if t < 40
                    else rng.permutation(E)[:k] for t in range(T)]).astype(np.int32)
    counts, offsets, perm, _ = oracle.dispatch(idx, E)
    y_perm = torch.full((T * k, m), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(layer.handle, layer.x, layer.x_dtype, T, m, p, E, k, to_device(perm), to_device(offsets),
                     y_perm, layer._ws, layer.ws_bytes)
    torch.cuda.synchronize()
    ref, _ = oracle.expert_rows(oracle.Experts.from_layer(L), L["x"], k, perm, offsets)
    got = y_perm.cpu().numpy()
    assert np.all(np.isfinite(got)), "rows left unwritten"
    assert_close(got, ref, "bf16", "y_perm")
    layer.close()


@pytest.mark.parametrize("w_dtype", ["bf16", "i8"])
@pytest.mark.parametrize("rows", ["0", "1"])
@pytest.mark.parametrize("sa", ["0", "1"])
@pytest.mark.parametrize("ks", ["1", "2"])
def test_skinny_epilogue_and_sharing(w_dtype, rows, sa, ks, tune):
    """Packed rows with the columns split over the waves: activations copied
    once per workgroup into LDS (sa=1) or loaded by every wave (sa=0); the down
    projection's unweighted rows summed by the combine kernel (rows=1, per
    reduction slice) or weighted rows added with atomics (rows=0); one or two
    reduction slices."""
    tune(ffn_path=M.MOE_PATH_SKINNY, skinny_mt=2, skinny_pack=1, skinny_splitk=-1,
         skinny_shared=1 if sa == "1" else -1, down_rows=1 if rows == "1" else -1, down_ksplit=int(ks))
    T, m, p, E, k = 70, 256, 384, 8, 2
    log(f"skinny epilogue w={w_dtype} rows={rows} sa={sa} ks={ks}")
    L = synth.make_layer(spec(T, m, p, E, k, "swiglu", w_dtype, seed=17 + 3 * int(ks), zipf=1.2, sw=0.05,
                              sr=0.05))
    layer = MoELayer(L)
    dbg = layer.debug_buffers()
    y = layer.forward(dbg=dbg)
    torch.cuda.synchronize()
    lg, idx_g, _, counts, _ = check_routing(L, dbg, T, E, k)
    ref, i_o, _, _ = oracle.forward_tokens(oracle.Experts.from_layer(L), L["x"], L["wg"], L["bias"], k,
                                           np.arange(T), logits=lg)
    assert np.array_equal(i_o, idx_g)
    assert_close(y_to_np(y), ref, w_dtype, "y")
    layer.close()


@pytest.mark.parametrize("w_dtype", ["bf16", "i8"])
def test_skinny_rows_repeat_is_bitwise(w_dtype, tune):
    """With unweighted rows and the combine kernel the layer has no atomics:
    two calls, with two reduction slices, give identical bits."""
    tune(ffn_path=M.MOE_PATH_SKINNY, down_ksplit=2)
    L = synth.make_layer(spec(200, 256, 384, 8, 2, "swiglu", w_dtype, seed=23, zipf=1.2, sw=0.05))
    layer = MoELayer(L)
    y1 = layer.forward().clone()
    y2 = layer.forward()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    layer.close()
