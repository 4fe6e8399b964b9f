"""The split decode launch against the CPU oracle.

With four M tiles and packed, shared activations, experts holding more than
one 64-row chunk are served by twelve-tile work items (192-row chunks) in the
same launch as the four-tile items of the others: for both projections by
default; moe_tuning.skinny_wide_down = -1 keeps the down projection on
four-tile items.
The cases force hot experts of every size class: 65..192 rows (one wide
chunk, ragged), several
wide chunks (over 192 rows), a mix of hot and cold experts, and none hot;
for the layer (unweighted rows and the combine kernel) and the expert-FFN
stage (unweighted rows), SwiGLU and ReLU.  Bars as in the other parity tests.
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
def _split(tune):
    tune(ffn_path=M.MOE_PATH_SKINNY, skinny_mt=4, skinny_pack=1)


# T, m, p, E, k, bias on the hot experts (None: routing as generated)
CASES = [
    (150, 256, 320, 8, 2, {0: 50.0}),             # expert 0: 150 rows, one ragged wide chunk
    (450, 192, 256, 8, 2, {0: 50.0}),             # expert 0: 450 rows, three wide chunks
    (300, 128, 384, 6, 2, {0: 50.0, 3: 0.5}),     # two hot experts beside cold ones
    (256, 256, 320, 16, 2, None),                 # Zipf-skewed routing as generated
    (40, 128, 192, 8, 2, None),                   # no expert above 64 rows
]


def _layer(T, m, p, E, k, bias, kind, seed):
    L = synth.make_layer(spec(T, m, p, E, k, kind, "bf16", seed=seed, zipf=1.2 if bias is None else None,
                              sw=0.05, sr=0.05))
    if bias:
        L["bias"] = np.zeros(E, np.float32)
        for e, b in bias.items():
            L["bias"][e] = b
    return L


@pytest.mark.parametrize("down", ["0", "1"])
@pytest.mark.parametrize("kind", ["swiglu", "relu"])
@pytest.mark.parametrize("T,m,p,E,k,bias", CASES)
def test_wide_layer(kind, T, m, p, E, k, bias, down, tune):
    """down=0 keeps the down projection on four-tile items."""
    tune(skinny_wide_down=1 if down == "1" else -1)
    log(f"wide layer kind={kind} down={down} T={T} m={m} p={p} E={E} k={k} bias={bias}")
    L = _layer(T, m, p, E, k, bias, kind, seed=T + p)
    layer = MoELayer(L)
    dbg = layer.debug_buffers()
    y = layer.forward(dbg=dbg)
    torch.cuda.synchronize()
    lg, idx_g, _, counts, _ = check_routing(L, dbg, T, E, k)
    log(f"  counts={counts.tolist()}")
    ref, i_o, _, _ = oracle.forward_tokens(oracle.Experts.from_layer(L), L["x"], L["wg"], L["bias"], k,
                                           np.arange(T), logits=lg)
    assert np.array_equal(i_o, idx_g)
    assert_close(y_to_np(y), ref, "bf16", "y")
    layer.close()


@pytest.mark.parametrize("down", ["0", "1"])
@pytest.mark.parametrize("kind", ["swiglu", "relu"])
@pytest.mark.parametrize("hot", [100, 300])
def test_wide_expert_ffn_stage(kind, hot, down, tune):
    """Expert 2 holds `hot` rows (one or two wide chunks); rows are unweighted."""
    tune(skinny_wide_down=1 if down == "1" else -1)
    T, m, p, E, k = 320, 128, 384, 6, 2
    L = synth.make_layer(spec(T, m, p, E, k, kind, "bf16", seed=hot, sw=0.05))
    layer = MoELayer(L)
    rng = np.random.default_rng(hot)
    idx = np.stack([np.concatenate([[2], rng.permutation([e for e in range(E) if e != 2])[:k - 1]]) if t < hot
                    else rng.permutation([e for e in range(E) if e != 2])[:k] for t in range(T)]).astype(np.int32)
    counts, offsets, perm, _ = oracle.dispatch(idx, E)
    assert counts[2] == hot
    y_perm = torch.full((T * k, m), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(layer.handle, layer.x, layer.x_dtype, T, m, p, E, k, to_device(perm), to_device(offsets),
                     y_perm, layer._ws, layer.ws_bytes)
    torch.cuda.synchronize()
    ref, _ = oracle.expert_rows(oracle.Experts.from_layer(L), L["x"], k, perm, offsets)
    got = y_perm.cpu().numpy()
    assert np.all(np.isfinite(got)), "rows left unwritten"
    assert_close(got, ref, "bf16", "y_perm")
    layer.close()


def test_wide_matches_narrow():
    """The split launch and the four-tile kernel alone agree to fp32 rounding
    (the two group a row's products into different accumulation orders)."""
    L = _layer(300, 128, 384, 6, 2, {0: 50.0, 3: 0.5}, "swiglu", seed=5)
    layer = MoELayer(L)
    y_split = layer.forward().float().clone()
    layer.set_tuning(dict(ffn_path=M.MOE_PATH_SKINNY, skinny_mt=4, skinny_pack=1, skinny_wide=-1))
    y_narrow = layer.forward().float()
    torch.cuda.synchronize()
    err = (y_split - y_narrow).abs().max().item()
    scale = y_narrow.abs().max().item()
    assert err <= 2 ** -7 * scale + 1e-6, (err, scale)
    layer.close()
