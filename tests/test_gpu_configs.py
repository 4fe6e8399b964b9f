"""The five measured layers at full size, in the launch configuration the
benchmark times, against the CPU oracle, and the int8, int4, fp8, fp8a8 and
i8a8 (8-bit weights and activations) Mixtral prefill layers (the grouped GEMM
with the weights' dequant fused, or on the fp8 / int8 matrix cores).

Routing and dispatch are checked in full.  Outputs are checked element by
element on every token of the tiny, decode, skewed and int8 layers.  On the
prefill layers (8192 tokens, the grouped GEMM) at least 512 tokens are
checked, chosen so that every (expert, row block) of the GEMM (256 rows; 128
for int4) contributes rows: the first and last row of every block (so each expert's ragged last
block and the first and last packed rows) and one inside it, topped up with
random tokens (tokens are independent rows).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from mixture_experts_layer_gemv_amd.layer import MoELayer

from _gpu import assert_close, check_routing, log, y_to_np

pytestmark = pytest.mark.gpu

BLOCK_ROWS = 256  # rows of one grouped-GEMM row block
PREFILL_MIN_TOKENS = 512


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def prefill_tokens(offsets, perm, k, T, seed, n_min=PREFILL_MIN_TOKENS, block=BLOCK_ROWS):
    """Tokens whose rows cover every (expert, row block): per block its first,
    last and one random row, then random tokens up to n_min.  Returns the
    sorted tokens and the number of blocks covered."""
    rng = np.random.default_rng(seed)
    toks, blocks = set(), 0
    E = len(offsets) - 1
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for r0 in range(lo, hi, block):
            r1 = min(r0 + block, hi) - 1
            for r in (r0, r1, int(rng.integers(r0, r1 + 1))):
                toks.add(int(perm[r]) // k)
            blocks += 1
    rest = [t for t in rng.permutation(T) if t not in toks]
    toks.update(int(t) for t in rest[:max(0, n_min - len(toks))])
    return np.array(sorted(toks)), blocks


@pytest.mark.parametrize("cfg", ["c1", "c2", "c3", "c4", "c5", "c7", "c8", "c11", "c12", "c14", "c15"])
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
    if sp.T >= 4096:  # prefill layers: the grouped GEMM
        offsets = dbg["offsets"].cpu().numpy()
        perm = dbg["perm"].cpu().numpy()
        bm = 128 if sp.w_dtype == "i4" else BLOCK_ROWS  # int4 runs 128-row blocks
        tokens, blocks = prefill_tokens(offsets, perm, sp.k, sp.T, seed=100 + sp.seed, block=bm)
        # every block of every expert has at least one row among the checked tokens
        rows = set(np.nonzero(np.isin(perm // sp.k, tokens))[0].tolist())
        for e in range(sp.E):
            for r0 in range(int(offsets[e]), int(offsets[e + 1]), bm):
                assert any(r in rows for r in range(r0, min(r0 + bm, int(offsets[e + 1])))), (e, r0)
        log(f"  checking {len(tokens)} tokens covering all {blocks} (expert, row block) pairs")
        assert len(tokens) >= PREFILL_MIN_TOKENS
    else:
        tokens = np.arange(sp.T)
    X = oracle.Experts.from_layer(L)
    ref, i_o, _, _ = oracle.forward_tokens(X, L["x"], L["wg"], L["bias"], sp.k, tokens, logits=lg)
    assert np.array_equal(i_o, idx_g[tokens])
    assert_close(y_to_np(y)[tokens], ref, sp.w_dtype, f"{cfg} y[{len(tokens)} tokens]")
    # A second call on the same handle: identical routing and, with no
    # atomics on these paths, identical output bits.
    dbg2 = layer.debug_buffers()
    y2 = layer.forward(dbg=dbg2)
    torch.cuda.synchronize()
    for key in dbg:
        assert torch.equal(dbg[key], dbg2[key]), key
    y1n, y2n = y_to_np(y), y_to_np(y2)
    assert np.max(np.abs(y1n - y2n)) <= 2.0**-7 * np.max(np.abs(y1n))
    layer.close()
    del L, X
