"""The five measured layers at full size, in the launch configuration the
benchmark times: routing and dispatch checked in full, outputs on sampled
tokens against the oracle (tokens are independent rows)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from mixture_experts_layer_gemv_amd.layer import MoELayer

from _gpu import assert_close, check_routing, log, y_to_np

pytestmark = pytest.mark.gpu

# tokens checked against the oracle per layer (all of them for the small ones)
SAMPLE = {"c1": None, "c2": None, "c3": 24, "c4": 12, "c5": 16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


@pytest.mark.parametrize("cfg", ["c1", "c2", "c3", "c4", "c5"])
def test_config_full_size(cfg):
    sp = synth.spec(cfg)
    log(f"config {cfg} ({sp.name}): T={sp.T} m={sp.m} p={sp.p} E={sp.E} k={sp.k} {sp.kind} "
        f"x={sp.x_dtype} w={sp.w_dtype}")
    L = synth.make_layer(sp)
    layer = MoELayer(L)
    dbg = layer.debug_buffers()
    y = layer.forward(dbg=dbg)
    torch.cuda.synchronize()
    lg, idx_g, w_g, counts, n_diff = check_routing(L, dbg, sp.T, sp.E, sp.k)
    log(f"  counts={counts.tolist()} tokens routed differently from oracle logits: {n_diff}")
    n = SAMPLE[cfg]
    if n is None:
        tokens = np.arange(sp.T)
    else:
        rng = np.random.default_rng(100 + sp.seed)
        tokens = np.sort(rng.choice(sp.T, size=n, replace=False))
        if cfg == "c3":  # make sure the hottest expert's rows are among the checked ones
            hot = int(np.argmax(counts))
            on_hot = np.nonzero(np.any(idx_g == hot, axis=1))[0]
            tokens = np.unique(np.concatenate([tokens, on_hot[:4], on_hot[-4:]]))
    X = oracle.Experts.from_layer(L)
    ref, i_o, _, _ = oracle.forward_tokens(X, L["x"], L["wg"], L["bias"], sp.k, tokens, logits=lg)
    assert np.array_equal(i_o, idx_g[tokens])
    assert_close(y_to_np(y)[tokens], ref, sp.w_dtype, f"{cfg} y[{len(tokens)} tokens]")
    # A second call on the same handle: identical routing; the output may
    # differ only by the order of the fp32 atomic adds of split reductions.
    dbg2 = layer.debug_buffers()
    y2 = layer.forward(dbg=dbg2)
    torch.cuda.synchronize()
    for key in dbg:
        assert torch.equal(dbg[key], dbg2[key]), key
    y1n, y2n = y_to_np(y), y_to_np(y2)
    assert np.max(np.abs(y1n - y2n)) <= 2.0**-7 * np.max(np.abs(y1n))
    layer.close()
    del L, X
