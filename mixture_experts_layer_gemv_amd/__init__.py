"""Python binding of libmoe_gemv.so (include/moe_gemv.h): argument marshalling only.

Every function has the C name and argument order.  Tensor arguments are
torch tensors on the GPU (or None for an optional pointer); they are passed
as raw device pointers.  ``stream`` defaults to torch's current stream.  A
non-zero status raises :class:`MoeError` carrying ``moe_last_error()``.

All computation happens in the HIP library: there is no Python or CPU
fallback, and importing the binding fails loudly when the library is absent.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_gemv.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_OOM = range(6)
MOE_F32, MOE_BF16, MOE_I8, MOE_I4, MOE_FP8, MOE_MXFP4, MOE_FP8A8, MOE_I8A8 = 0, 1, 2, 3, 4, 5, 6, 7
MOE_MLP_RELU, MOE_SWIGLU = 0, 1
MOE_ROUTE_LOGITS_IN = 1
MOE_NORM_NONE, MOE_NORM_LAYER, MOE_NORM_RMS = 0, 1, 2
MOE_MAX_EXPERTS = 64
MOE_PATH_AUTO, MOE_PATH_SKINNY, MOE_PATH_GEMM = 0, 1, 2
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE",
                4: "MOE_ERR_HIP", 5: "MOE_ERR_OOM"}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class moe_tuning(ctypes.Structure):
    """struct moe_tuning: 0 is "automatic" in every field, switches are 1 / -1."""
    _fields_ = [(n, ctypes.c_int) for n in (
        "ffn_path", "skinny_mt", "skinny_pack", "skinny_splitk", "skinny_shared", "skinny_wide", "skinny_wide_down",
        "up_ct", "down_ct", "down_ksplit", "down_rows", "gemm_cg", "gemm_skip", "route_quant")]


def tuning(**fields) -> moe_tuning:
    """A moe_tuning with the given fields set (the rest automatic)."""
    t = moe_tuning()
    for k, v in fields.items():
        if not hasattr(t, k):
            raise KeyError(k)
        setattr(t, k, int(v))
    return t


_lib = None

_vp, _i32, _u32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t
_SIGS = {
    "moe_last_error": ([], ctypes.c_char_p),
    "moe_abi_version": ([], _i32),
    "moe_weights_create": ([_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                            ctypes.POINTER(_vp)], _i32),
    "moe_weights_destroy": ([_vp], _i32),
    "moe_weights_offload": ([_vp, _i32, _vp], _i32),
    "moe_weights_offload_stats": ([_vp, ctypes.POINTER(ctypes.c_longlong), ctypes.POINTER(ctypes.c_longlong),
                                   ctypes.POINTER(ctypes.c_longlong)], _i32),
    "moe_workspace_size": ([_vp, _i32, _i32, ctypes.POINTER(_sz)], _i32),
    "moe_weights_set_tuning": ([_vp, ctypes.POINTER(moe_tuning)], _i32),
    "moe_weights_get_tuning": ([_vp, ctypes.POINTER(moe_tuning)], _i32),
    "moe_workspace_size_for": ([_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(moe_tuning), _i32, _i32,
                                ctypes.POINTER(_sz)], _i32),
    "moe_route_topk": ([_vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _u32, _vp, _vp, _vp, _vp], _i32),
    "moe_dispatch": ([_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp], _i32),
    "moe_expert_ffn": ([_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "moe_combine": ([_vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp], _i32),
    "moe_quantize_rows_e4m3": ([_vp, _i32, _i32, _vp, _vp, _vp], _i32),
    "moe_quantize_rows_i8": ([_vp, _i32, _i32, _vp, _vp, _vp], _i32),
    "moe_layer_forward": ([_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _sz,
                           _vp, _vp, _vp, _vp, _vp, _vp, _vp], _i32),
    "moe_layer_forward_fused": ([_vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, ctypes.c_float, _vp, _i32, _i32, _i32,
                                 _i32, _i32, _vp, _i32, _vp, _sz, _vp, _vp, _vp, _vp, _vp], _i32),
    "moe_layer_graph_create": ([_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _sz,
                                ctypes.POINTER(_vp)], _i32),
    "moe_graph_launch": ([_vp, _vp], _i32),
    "moe_layer_forward_noalloc": ([_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _i32, _vp], _i32),
    "moe_graph_destroy": ([_vp], _i32),
    "moe_profile_begin": ([_i32], _i32),
    "moe_profile_end": ([], _i32),
    "moe_profile_query": ([ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i32)], _i32),
}


def lib():
    """Load libmoe_gemv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(or python mixture_experts_layer_gemv_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, rc):
    if rc != MOE_OK:
        raise MoeError(fn, rc, lib().moe_last_error().decode())


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_weights_create(m, p, E, kind, w_dtype, w1, w_up, w2, s1=None, s_up=None, s2=None, stream=None):
    h = _vp()
    _check("moe_weights_create", lib().moe_weights_create(m, p, E, kind, w_dtype, _p(w1), _p(w_up), _p(w2), _p(s1),
                                                          _p(s_up), _p(s2), _s(stream), ctypes.byref(h)))
    return h


def moe_weights_destroy(w):
    _check("moe_weights_destroy", lib().moe_weights_destroy(w))


def moe_weights_offload(w, slots, stream=None):
    _check("moe_weights_offload", lib().moe_weights_offload(w, slots, _s(stream)))


def moe_weights_offload_stats(w):
    """(hits, misses, bytes copied host -> device) of an offloaded handle."""
    h, m_, b = ctypes.c_longlong(), ctypes.c_longlong(), ctypes.c_longlong()
    _check("moe_weights_offload_stats", lib().moe_weights_offload_stats(w, ctypes.byref(h), ctypes.byref(m_),
                                                                        ctypes.byref(b)))
    return h.value, m_.value, b.value


def moe_workspace_size(w, T, k) -> int:
    n = _sz()
    _check("moe_workspace_size", lib().moe_workspace_size(w, T, k, ctypes.byref(n)))
    return n.value


def moe_weights_set_tuning(w, t=None):
    """t: a moe_tuning, a dict of its fields, or None (all automatic)."""
    if isinstance(t, dict):
        t = tuning(**t)
    _check("moe_weights_set_tuning", lib().moe_weights_set_tuning(w, None if t is None else ctypes.byref(t)))


def moe_weights_get_tuning(w) -> moe_tuning:
    t = moe_tuning()
    _check("moe_weights_get_tuning", lib().moe_weights_get_tuning(w, ctypes.byref(t)))
    return t


def moe_workspace_size_for(m, p, E, kind, w_dtype, t, T, k) -> int:
    if isinstance(t, dict):
        t = tuning(**t)
    n = _sz()
    _check("moe_workspace_size_for", lib().moe_workspace_size_for(
        m, p, E, kind, w_dtype, None if t is None else ctypes.byref(t), T, k, ctypes.byref(n)))
    return n.value


def moe_route_topk(x, x_dtype, w_router, b_router, T, m, E, k, flags, logits, topk_idx, topk_w, stream=None):
    _check("moe_route_topk", lib().moe_route_topk(_p(x), x_dtype, _p(w_router), _p(b_router), T, m, E, k, flags,
                                                  _p(logits), _p(topk_idx), _p(topk_w), _s(stream)))


def moe_dispatch(topk_idx, T, E, k, counts, offsets, perm, inv_perm, stream=None):
    _check("moe_dispatch", lib().moe_dispatch(_p(topk_idx), T, E, k, _p(counts), _p(offsets), _p(perm),
                                              _p(inv_perm), _s(stream)))


def moe_expert_ffn(w, x, x_dtype, T, m, p, E, k, perm, offsets, y_perm, workspace, ws_bytes, stream=None):
    _check("moe_expert_ffn", lib().moe_expert_ffn(w, _p(x), x_dtype, T, m, p, E, k, _p(perm), _p(offsets),
                                                  _p(y_perm), _p(workspace), ws_bytes, _s(stream)))


def moe_combine(y_perm, inv_perm, topk_w, T, m, k, y, y_dtype, stream=None):
    _check("moe_combine", lib().moe_combine(_p(y_perm), _p(inv_perm), _p(topk_w), T, m, k, _p(y), y_dtype,
                                            _s(stream)))


def moe_quantize_rows_e4m3(x, T, m, xq, scale, stream=None):
    _check("moe_quantize_rows_e4m3", lib().moe_quantize_rows_e4m3(_p(x), T, m, _p(xq), _p(scale), _s(stream)))


def moe_quantize_rows_i8(x, T, m, xq, scale, stream=None):
    _check("moe_quantize_rows_i8", lib().moe_quantize_rows_i8(_p(x), T, m, _p(xq), _p(scale), _s(stream)))


def moe_layer_forward(w, w_router, b_router, x, x_dtype, T, m, p, E, k, y, y_dtype, workspace, ws_bytes,
                      dbg_topk_idx=None, dbg_topk_w=None, dbg_logits=None, dbg_counts=None, dbg_offsets=None,
                      dbg_perm=None, stream=None):
    _check("moe_layer_forward", lib().moe_layer_forward(
        w, _p(w_router), _p(b_router), _p(x), x_dtype, T, m, p, E, k, _p(y), y_dtype, _p(workspace), ws_bytes,
        _p(dbg_topk_idx), _p(dbg_topk_w), _p(dbg_logits), _p(dbg_counts), _p(dbg_offsets), _p(dbg_perm),
        _s(stream)))


def moe_layer_forward_fused(w, w_router, b_router, x, x_dtype, norm, gamma, beta, eps, residual, T, m, p, E, k, y,
                            y_dtype, workspace, ws_bytes, x_norm=None, dbg_topk_idx=None, dbg_topk_w=None,
                            dbg_logits=None, stream=None):
    _check("moe_layer_forward_fused", lib().moe_layer_forward_fused(
        w, _p(w_router), _p(b_router), _p(x), x_dtype, norm, _p(gamma), _p(beta), float(eps), _p(residual), T, m, p,
        E, k, _p(y), y_dtype, _p(workspace), ws_bytes, _p(x_norm), _p(dbg_topk_idx), _p(dbg_topk_w),
        _p(dbg_logits), _s(stream)))


def moe_layer_graph_create(w, w_router, b_router, x, x_dtype, T, m, p, E, k, y, y_dtype, workspace, ws_bytes):
    """Returns the graph handle (an int)."""
    g = _vp()
    _check("moe_layer_graph_create", lib().moe_layer_graph_create(
        w, _p(w_router), _p(b_router), _p(x), x_dtype, T, m, p, E, k, _p(y), y_dtype, _p(workspace), ws_bytes,
        ctypes.byref(g)))
    return g.value


def moe_layer_forward_noalloc(w, w_router, b_router, x, x_dtype, T, m, p, E, k, y, y_dtype, stream=None):
    _check("moe_layer_forward_noalloc", lib().moe_layer_forward_noalloc(
        w, _p(w_router), _p(b_router), _p(x), x_dtype, T, m, p, E, k, _p(y), y_dtype, _s(stream)))


def moe_graph_launch(g, stream=None):
    _check("moe_graph_launch", lib().moe_graph_launch(g, _s(stream)))


def moe_graph_destroy(g):
    _check("moe_graph_destroy", lib().moe_graph_destroy(g))


def moe_profile_begin(max_launches: int):
    _check("moe_profile_begin", lib().moe_profile_begin(max_launches))


def moe_profile_end():
    _check("moe_profile_end", lib().moe_profile_end())


def moe_profile_query(kernel: str):
    ms, n = ctypes.c_double(), _i32()
    _check("moe_profile_query", lib().moe_profile_query(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
