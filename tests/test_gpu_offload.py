"""Host-resident experts (moe_weights_offload) against the device-resident
forward and the CPU oracle.

After moe_weights_offload the experts live in pinned host memory and a
forward streams the touched ones into a few device slots (an LRU expert
cache), overlapping each copy with the compute of the experts before it.
Each expert runs the same kernels with the layer's own launch choices, so
the output must equal the device-resident forward bit for bit on every path
without atomics, and stay at the oracle's parity bar.  Also checked: the
cache counters over repeated and changing batches, the expert-FFN stage, and
the refusals (graph capture, the allocation-free forward, fp32 weights, bad
slot counts).
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


# name, (T, m, p, E, k, kind, w_dtype, zipf)
CASES = [
    ("decode_bf16", (16, 512, 1024, 8, 2, "swiglu", "bf16", None)),
    ("decode_int8", (64, 512, 1024, 8, 2, "swiglu", "i8", None)),
    ("decode_int4", (40, 256, 512, 8, 2, "swiglu", "i4", None)),
    ("decode_fp8", (40, 256, 512, 8, 2, "swiglu", "fp8", None)),
    ("decode_mxfp4", (40, 256, 512, 8, 2, "relu", "mxfp4", None)),
    ("skewed_split", (256, 256, 640, 16, 2, "swiglu", "bf16", 1.2)),
    ("relu_bf16", (40, 256, 512, 8, 2, "relu", "bf16", None)),
    ("prefill_gemm", (1536, 256, 512, 4, 2, "swiglu", "bf16", None)),
    ("prefill_gemm_int4", (1536, 256, 512, 4, 2, "swiglu", "i4", None)),
    ("prefill_gemm_mxfp4", (1536, 256, 512, 4, 2, "swiglu", "mxfp4", None)),  # one expert expanded at a time
]


@pytest.mark.parametrize("slots", [1, 2, "E"])
@pytest.mark.parametrize("name,shape", CASES, ids=[c[0] for c in CASES])
def test_offloaded_layer_matches_resident(name, shape, slots):
    T, m, p, E, k, kind, wd, zipf = shape
    slots = E if slots == "E" else slots
    log(f"offload {name} slots={slots}: T={T} m={m} p={p} E={E} k={k} {kind} {wd}")
    L = synth.make_layer(spec(T, m, p, E, k, kind, wd, seed=T + p + 5, zipf=zipf, sw=0.05, sr=0.05))
    resident = MoELayer(L)
    y_res = resident.forward().clone()
    torch.cuda.synchronize()
    resident.close()
    layer = MoELayer(L)
    layer.offload(slots)
    for rep in range(2):  # a cold and a warm forward
        dbg = layer.debug_buffers()
        y = layer.forward(dbg=dbg)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_res.view(torch.int16)), f"{name} rep {rep}: differs from resident"
    lg, idx_g, _, counts, _ = check_routing(L, dbg, T, E, k)
    ref, _, _, _ = oracle.forward_tokens(oracle.Experts.from_layer(L), L["x"], L["wg"], L["bias"], k, np.arange(T),
                                         logits=lg)
    assert_close(y_to_np(y), ref, "bf16", f"{name} offloaded vs oracle")
    hits, misses, nbytes = M.moe_weights_offload_stats(layer.handle)
    touched = int(np.sum(counts > 0))
    log(f"  touched={touched} hits={hits} misses={misses} bytes={nbytes}")
    assert hits + misses == 2 * touched
    if slots >= touched:
        assert misses == touched and hits == touched  # the warm forward finds every expert cached
    expert_bytes = nbytes // max(misses, 1)
    assert nbytes == misses * expert_bytes
    layer.close()


def test_cache_follows_changing_batches():
    """Batches routed to different experts: slots are refilled least recently
    used first, every forward matches the resident one and the counters add
    up."""
    T, m, p, E, k = 24, 256, 512, 8, 1
    L = synth.make_layer(spec(T, m, p, E, k, "swiglu", "bf16", seed=31, sw=0.05, sr=0.05))
    resident = MoELayer(L)
    layer = MoELayer(L)
    layer.offload(3)
    total_touched = 0
    for b, hot in enumerate([(0, 1), (0, 1), (2, 3), (0, 4), (5, 6, 7), (5, 6, 7)]):
        bias = np.full(E, -50.0, np.float32)
        bias[list(hot)] = 0.0
        b_dev = to_device(bias)
        resident.bias = b_dev
        layer.bias = b_dev
        y_res = resident.forward().clone()
        dbg = layer.debug_buffers()
        y = layer.forward(dbg=dbg)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_res.view(torch.int16)), f"batch {b}"
        counts = dbg["counts"].cpu().numpy()
        assert set(np.nonzero(counts)[0].tolist()) <= set(hot)
        total_touched += int(np.sum(counts > 0))
    hits, misses, _ = M.moe_weights_offload_stats(layer.handle)
    log(f"  hits={hits} misses={misses}")
    assert hits + misses == total_touched
    assert hits >= 2  # batches 2 and 6 repeat the experts of their predecessors
    resident.close()
    layer.close()


def test_offloaded_expert_ffn_stage():
    T, m, p, E, k = 50, 256, 384, 8, 2
    L = synth.make_layer(spec(T, m, p, E, k, "swiglu", "i8", seed=8, sw=0.05))
    rng = np.random.default_rng(4)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, _ = oracle.dispatch(idx, E)
    outs = []
    for off in (False, True):
        layer = MoELayer(L)
        if off:
            layer.offload(2)
        y_perm = torch.full((T * k, m), float("nan"), dtype=torch.float32, device="cuda")
        M.moe_expert_ffn(layer.handle, layer.x, layer.x_dtype, T, m, p, E, k, to_device(perm), to_device(offsets),
                         y_perm, layer.ensure_workspace(T), layer.ws_bytes)
        torch.cuda.synchronize()
        outs.append(y_perm.cpu().numpy())
        layer.close()
    assert np.array_equal(outs[0], outs[1])
    ref, _ = oracle.expert_rows(oracle.Experts.from_layer(L), L["x"], k, perm, offsets)
    assert_close(outs[1], ref, "bf16", "y_perm offloaded")


def test_offload_refusals():
    L = synth.make_layer(spec(8, 256, 512, 8, 2, "swiglu", "bf16", seed=2))
    layer = MoELayer(L)
    for bad in (0, 9):
        with pytest.raises(M.MoeError) as ei:
            layer.offload(bad)
        assert ei.value.status == M.MOE_ERR_INVALID_ARG
    layer.offload(4)
    with pytest.raises(M.MoeError) as ei:
        layer.offload(4)
    assert ei.value.status == M.MOE_ERR_INVALID_ARG
    with pytest.raises(M.MoeError) as ei:
        layer.capture()
    assert ei.value.status == M.MOE_ERR_UNSUPPORTED
    y = layer.new_output()
    with pytest.raises(M.MoeError) as ei:
        M.moe_layer_forward_noalloc(layer.handle, layer.wg, layer.bias, layer.x, layer.x_dtype, 8, 256, 512, 8, 2, y,
                                    layer.y_dtype)
    assert ei.value.status == M.MOE_ERR_UNSUPPORTED
    layer.forward(y=y)  # still usable after the refusals
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()
    layer.close()
    L32 = synth.make_layer(spec(8, 256, 512, 8, 2, "relu", "f32", seed=2))
    layer = MoELayer(L32)
    with pytest.raises(M.MoeError) as ei:
        layer.offload(2)
    assert ei.value.status == M.MOE_ERR_UNSUPPORTED
    layer.close()
