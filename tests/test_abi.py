"""The C ABI library loads, exports what include/moe_gemv.h declares, and
rejects bad arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_gemv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(moe_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    import mixture_experts_layer_gemv_amd as M

    if not os.path.exists(M.LIB_PATH):
        pytest.fail("libmoe_gemv.so is not built (run __graft_entry__.build())")
    return M


def test_header_declares_the_boundary():
    names = _declared()
    for fn in ["moe_route_topk", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_layer_forward",
               "moe_weights_create", "moe_weights_destroy", "moe_workspace_size", "moe_last_error"]:
        assert fn in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s+(moe_\w+)$", out, flags=re.M))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    L = lib.lib()
    for n in _declared():
        assert hasattr(L, n)
    assert lib.moe_abi_version() == 2


def test_binding_names_match_header(lib):
    for n in _declared():
        assert callable(getattr(lib, n)), n


FAKE = 0x7F0000000000  # never dereferenced: every case below fails validation first


def _rc(fn, *args):
    return fn(*args)


def test_weights_create_validation(lib):
    L = lib.lib()
    out = ctypes.c_void_p()
    Z = None
    # out == NULL
    assert L.moe_weights_create(64, 64, 8, 1, 1, FAKE, FAKE, FAKE, Z, Z, Z, Z, None) == lib.MOE_ERR_INVALID_ARG
    cases = [
        ((64, 64, 65, 1, 1, FAKE, FAKE, FAKE, Z, Z, Z), lib.MOE_ERR_UNSUPPORTED),  # E > 64
        ((64, 64, 0, 1, 1, FAKE, FAKE, FAKE, Z, Z, Z), lib.MOE_ERR_INVALID_ARG),  # E < 1
        ((100, 64, 8, 1, 1, FAKE, FAKE, FAKE, Z, Z, Z), lib.MOE_ERR_UNSUPPORTED),  # m % 64
        ((64, 96, 8, 1, 1, FAKE, FAKE, FAKE, Z, Z, Z), lib.MOE_ERR_UNSUPPORTED),  # p % 64
        ((64, 64, 8, 1, 8, FAKE, FAKE, FAKE, Z, Z, Z), lib.MOE_ERR_UNSUPPORTED),  # dtype
        ((64, 64, 8, 5, 1, FAKE, FAKE, FAKE, Z, Z, Z), lib.MOE_ERR_INVALID_ARG),  # kind
        ((64, 64, 8, 1, 1, FAKE, Z, FAKE, Z, Z, Z), lib.MOE_ERR_INVALID_ARG),  # SwiGLU without w_up
        ((64, 64, 8, 0, 1, FAKE, FAKE, FAKE, Z, Z, Z), lib.MOE_ERR_INVALID_ARG),  # ReLU with w_up
        ((64, 64, 8, 1, 2, FAKE, FAKE, FAKE, Z, Z, Z), lib.MOE_ERR_INVALID_ARG),  # int8 without scales
        ((64, 64, 8, 1, 1, FAKE, FAKE, FAKE, FAKE, Z, Z), lib.MOE_ERR_INVALID_ARG),  # scales for bf16
        ((64, 64, 8, 1, 1, FAKE + 2, FAKE, FAKE, Z, Z, Z), lib.MOE_ERR_INVALID_ARG),  # misaligned
    ]
    for args, want in cases:
        rc = L.moe_weights_create(*args, None, ctypes.byref(out))
        assert rc == want, (args, rc, lib.moe_last_error())
        assert out.value is None
        assert lib.moe_last_error() != ""


def test_stage_validation_without_gpu(lib):
    L = lib.lib()
    Z = None
    # route: k > E, E > 64, bad flags, NULL outputs, misaligned x
    assert L.moe_route_topk(FAKE, 1, FAKE, Z, 4, 64, 8, 9, 0, Z, FAKE, FAKE, Z) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_route_topk(FAKE, 1, FAKE, Z, 4, 64, 65, 2, 0, Z, FAKE, FAKE, Z) == lib.MOE_ERR_UNSUPPORTED
    assert L.moe_route_topk(FAKE, 1, FAKE, Z, 4, 64, 8, 2, 4, Z, FAKE, FAKE, Z) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_route_topk(FAKE, 1, FAKE, Z, 4, 64, 8, 2, 0, Z, Z, FAKE, Z) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_route_topk(FAKE, 2, FAKE, Z, 4, 64, 8, 2, 0, Z, FAKE, FAKE, Z) == lib.MOE_ERR_UNSUPPORTED
    assert L.moe_route_topk(FAKE + 8, 1, FAKE, Z, 4, 64, 8, 2, 0, Z, FAKE, FAKE, Z) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_route_topk(Z, 1, Z, Z, 4, 64, 8, 2, 1, Z, FAKE, FAKE, Z) == lib.MOE_ERR_INVALID_ARG  # LOGITS_IN
    assert L.moe_route_topk(FAKE, 1, FAKE, Z, -1, 64, 8, 2, 0, Z, FAKE, FAKE, Z) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_route_topk(FAKE, 1, FAKE, Z, 0, 64, 8, 2, 0, Z, FAKE, FAKE, Z) == lib.MOE_OK  # T = 0: no-op
    # dispatch
    assert L.moe_dispatch(FAKE, 4, 8, 0, FAKE, FAKE, FAKE, FAKE, Z) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_dispatch(FAKE, 4, 8, 2, Z, FAKE, FAKE, FAKE, Z) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_dispatch(FAKE, 2**30, 8, 4, FAKE, FAKE, FAKE, FAKE, Z) == lib.MOE_ERR_UNSUPPORTED
    # combine
    assert L.moe_combine(FAKE, FAKE, FAKE, 4, 96, 2, FAKE, 1, Z) == lib.MOE_ERR_UNSUPPORTED
    assert L.moe_combine(FAKE, FAKE, FAKE, 4, 64, 2, FAKE, 2, Z) == lib.MOE_ERR_UNSUPPORTED
    assert L.moe_combine(Z, FAKE, FAKE, 4, 64, 2, FAKE, 1, Z) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_combine(FAKE, FAKE, FAKE, 0, 64, 2, FAKE, 1, Z) == lib.MOE_OK
    # the fp8-activation quantisation step
    assert L.moe_quantize_rows_e4m3(FAKE, 4, 96, FAKE, FAKE, Z) == lib.MOE_ERR_UNSUPPORTED
    assert L.moe_quantize_rows_e4m3(Z, 4, 64, FAKE, FAKE, Z) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_rows_e4m3(FAKE + 8, 4, 64, FAKE, FAKE, Z) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_rows_e4m3(FAKE, -1, 64, FAKE, FAKE, Z) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_quantize_rows_e4m3(FAKE, 0, 64, FAKE, FAKE, Z) == lib.MOE_OK
    assert L.moe_quantize_rows_i8(FAKE, 4, 96, FAKE, FAKE, Z) == lib.MOE_ERR_UNSUPPORTED
    assert L.moe_quantize_rows_i8(FAKE, 4, 64, Z, FAKE, Z) == lib.MOE_ERR_INVALID_ARG
    # handle-based calls with a NULL handle
    assert L.moe_expert_ffn(Z, FAKE, 1, 4, 64, 64, 8, 2, FAKE, FAKE, FAKE, FAKE, 1 << 20, Z) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward(Z, FAKE, Z, FAKE, 1, 4, 64, 64, 8, 2, FAKE, 1, FAKE, 1 << 20,
                               Z, Z, Z, Z, Z, Z, Z) == lib.MOE_ERR_INVALID_ARG
    n = ctypes.c_size_t()
    assert L.moe_workspace_size(Z, 4, 2, ctypes.byref(n)) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_weights_destroy(Z) == lib.MOE_OK


def test_profile_query_is_host_only(lib):
    ms, n = lib.moe_profile_query("ffn_up")
    assert (ms, n) == (0.0, 0)
    with pytest.raises(lib.MoeError):
        lib.moe_profile_end()  # never started


def test_binding_raises_with_message(lib):
    with pytest.raises(lib.MoeError) as ei:
        lib.moe_combine(FAKE, FAKE, FAKE, 4, 96, 2, FAKE, 1, stream=0)
    assert ei.value.status == lib.MOE_ERR_UNSUPPORTED and "multiple of 64" in ei.value.message


# the five measured layers and the int4 decode layer: (m, p, E, kind, w_dtype, T, k)
LAYERS = [(256, 512, 8, 0, 0, 32, 2), (4096, 14336, 8, 1, 1, 16, 2), (4096, 6400, 16, 1, 1, 256, 2),
          (4096, 14336, 8, 1, 1, 8192, 2), (4096, 14336, 8, 1, 2, 64, 2), (4096, 14336, 8, 1, 3, 64, 2)]
# knobs that once tuned the launch plan through the environment
STALE_ENV = {"MOE_FFN_PATH": "s", "MOE_SKINNY_MT": "1", "MOE_SKINNY_PACK": "0", "MOE_SKINNY_WAVES": "k",
             "MOE_DOWN_KSPLIT": "4", "MOE_DOWN_ROWS": "0", "MOE_HOT_ROWS": "3", "MOE_GEMM_CG": "2"}


def test_workspace_size_ignores_the_environment(lib, monkeypatch):
    """The workspace (and the launch plan it is carved for) is a function of
    the layer, its tuning, T and k only."""
    before = [lib.moe_workspace_size_for(*L[:5], None, *L[5:]) for L in LAYERS]
    for k, v in STALE_ENV.items():
        monkeypatch.setenv(k, v)
    after = [lib.moe_workspace_size_for(*L[:5], None, *L[5:]) for L in LAYERS]
    assert before == after
    assert all(b > 0 for b in before)
    # an explicit tuning does change the plan: the prefill layer on the
    # decode kernels with gathered (unpacked) rows
    t = lib.tuning(ffn_path=lib.MOE_PATH_SKINNY, skinny_mt=1)
    assert lib.moe_workspace_size_for(*LAYERS[3][:5], t, *LAYERS[3][5:]) != before[3]


def test_tuning_validation(lib):
    L = lib.lib()
    n = ctypes.c_size_t()
    for bad in [dict(ffn_path=3), dict(skinny_mt=3), dict(up_ct=8), dict(skinny_pack=2), dict(down_rows=-2),
                dict(down_ksplit=-1), dict(gemm_cg=-4), dict(gemm_skip=5), dict(route_quant=2)]:
        t = lib.tuning(**bad)
        rc = L.moe_workspace_size_for(4096, 14336, 8, 1, 1, ctypes.byref(t), 16, 2, ctypes.byref(n))
        assert rc == lib.MOE_ERR_INVALID_ARG, (bad, rc)
    assert L.moe_weights_set_tuning(None, None) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_weights_get_tuning(None, None) == lib.MOE_ERR_INVALID_ARG
    # shape errors of the host-only sizing
    assert L.moe_workspace_size_for(100, 64, 8, 1, 1, None, 4, 2, ctypes.byref(n)) == lib.MOE_ERR_UNSUPPORTED
    assert L.moe_workspace_size_for(128, 192, 8, 1, 3, None, 4, 2, ctypes.byref(n)) == lib.MOE_ERR_UNSUPPORTED
    assert L.moe_workspace_size_for(64, 64, 8, 1, 1, None, 4, 9, ctypes.byref(n)) == lib.MOE_ERR_INVALID_ARG
    assert L.moe_workspace_size_for(64, 64, 8, 1, 1, None, 4, 2, None) == lib.MOE_ERR_INVALID_ARG
    assert lib.moe_workspace_size_for(64, 64, 8, 1, 1, None, 0, 2) > 0
    # fp8 activations add the quantised rows (bf16) and the per-token scales
    fp8 = lib.moe_workspace_size_for(4096, 14336, 8, 1, lib.MOE_FP8, None, 64, 2)
    fp8a8 = lib.moe_workspace_size_for(4096, 14336, 8, 1, lib.MOE_FP8A8, None, 64, 2)
    assert fp8a8 - fp8 == 64 * 4096 * 2 + 256
    i8a8 = lib.moe_workspace_size_for(4096, 14336, 8, 1, lib.MOE_I8A8, None, 64, 2)
    assert i8a8 - lib.moe_workspace_size_for(4096, 14336, 8, 1, lib.MOE_I8, None, 64, 2) == 64 * 4096 * 2 + 256
    assert L.moe_workspace_size_for(64, 64, 8, 1, 8, None, 4, 2, ctypes.byref(n)) == lib.MOE_ERR_UNSUPPORTED
