"""CPU oracle for one MoE-layer forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  The product path (the HIP library and its
binding) never does.  The arithmetic lives in ``moe_oracle.c`` (plain C,
double precision), which shares no code with the HIP library; this module
only marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

F32, BF16, I8, FP8, MXFP4, FP8A8, I8A8 = 0, 1, 2, 3, 4, 5, 6
RELU, SWIGLU = 0, 1
MAX_E = 64
# weight dtypes by name (int4 weights are int8 values in [-7, 7] to the oracle;
# "fp8a8" / "i8a8": fp8 / int8 weights with each token's expert input
# quantised to E4M3 / int8)
_DT = {"f32": F32, "bf16": BF16, "i8": I8, "i4": I8, "fp8": FP8, "mxfp4": MXFP4, "fp8a8": FP8A8, "i8a8": I8A8}
_KIND = {"relu": RELU, "swiglu": SWIGLU}


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(
        ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-I", _HERE, "-o", tmp, _SRC, "-lm"],
        check=True,
    )
    os.replace(tmp, _LIB)
    return _LIB


class _Experts(ctypes.Structure):
    _fields_ = [
        ("m", ctypes.c_int), ("p", ctypes.c_int), ("E", ctypes.c_int),
        ("kind", ctypes.c_int), ("w_dtype", ctypes.c_int),
        ("w1", ctypes.c_void_p), ("w3", ctypes.c_void_p), ("w2", ctypes.c_void_p),
        ("s1", ctypes.c_void_p), ("s3", ctypes.c_void_p), ("s2", ctypes.c_void_p),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        P = ctypes.POINTER(_Experts)
        L.orc_router_logits.argtypes = [vp, i32, vp, vp, i32, i32, i32, vp]
        L.orc_topk.argtypes = [vp, i32, i32, i32, vp, vp]
        L.orc_dispatch.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
        L.orc_expert_apply.argtypes = [P, i32, vp, vp, vp]
        L.orc_expert_rows.argtypes = [P, vp, i32, i32, i32, vp, vp, vp, i32, vp, vp]
        L.orc_combine.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp]
        L.orc_forward_tokens.argtypes = [P, vp, i32, vp, vp, vp, i32, i32, vp, i32, vp, vp, vp, vp]
        L.orc_dense_masked.argtypes = [P, vp, i32, vp, vp, i32, i32, vp]
        L.orc_max_threads.argtypes = []
        L.orc_set_threads.argtypes = [i32]
        L.orc_set_threads.restype = None
        L.orc_norm.argtypes = [vp, i32, i32, i32, i32, vp, vp, ctypes.c_double, vp]
        i64 = ctypes.c_int64
        L.orc_weight_value.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, ctypes.POINTER(ctypes.c_double)]
        L.orc_e4m3_encode.argtypes = [vp, i64, vp]
        L.orc_quant_rows_e4m3.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.orc_quant_rows_i8.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.orc_max_threads.restype = ctypes.c_int
        for f in ("orc_weight_value", "orc_norm", "orc_router_logits", "orc_topk", "orc_dispatch", "orc_expert_apply", "orc_expert_rows",
                  "orc_combine", "orc_forward_tokens", "orc_dense_masked"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def max_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().orc_max_threads())


def set_threads(n: int) -> None:
    """Threads of the oracle's later parallel loops."""
    lib().orc_set_threads(int(n))


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))
    return a


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def _xdt(x):
    return BF16 if x.dtype == np.uint16 else F32


class Experts:
    """Expert weights of one layer in canonical layout (see synth).  w_dtype
    ("fp8", "fp8a8" or "mxfp4") names the uint8 weight formats; the others
    follow from the arrays' dtypes (fp32, bf16 as uint16, int8)."""

    def __init__(self, kind, w1, w2, w3=None, s1=None, s2=None, s3=None, w_dtype=None):
        self.kind = kind
        self.w1, self.w2, self.w3 = _c(w1), _c(w2), _c(w3)
        sdt = np.uint8 if w_dtype == "mxfp4" else np.float32
        self.s1, self.s2, self.s3 = _c(s1, sdt), _c(s2, sdt), _c(s3, sdt)
        E, m, p = self.w1.shape
        assert self.w2.shape == (E, p, m)
        if w_dtype in ("fp8", "fp8a8", "mxfp4"):
            assert self.w1.dtype == np.uint8
            dt = _DT[w_dtype]
        elif self.w1.dtype == np.float32:
            dt = F32
        elif self.w1.dtype == np.uint16:
            dt = BF16
        elif self.w1.dtype == np.int8:
            dt = I8A8 if w_dtype == "i8a8" else I8
        else:
            raise TypeError(self.w1.dtype)
        self.E, self.m, self.p, self.w_dtype = E, m, p, dt
        self._s = _Experts(m, p, E, _KIND[kind], dt, _ptr(self.w1), _ptr(self.w3), _ptr(self.w2),
                           _ptr(self.s1), _ptr(self.s3), _ptr(self.s2))

    @classmethod
    def from_layer(cls, layer):
        sp = layer["spec"]
        return cls(sp.kind, layer["w1"], layer["w2"], layer["w3"], layer["s1"], layer["s2"], layer["s3"],
                   w_dtype=sp.w_dtype)

    def param_bytes(self) -> int:
        """Bytes of one expert's weight matrices as stored."""
        nmat = 3 if self.kind == "swiglu" else 2
        return nmat * self.m * self.p * self.w1.itemsize


def weight_value(w, s, dtype, e, k, n):
    """Decoded weight (e, k, n) of a [E][K][N] projection w in dtype (a name of
    _DT) with its scales s, as the oracle's expert uses it."""
    w = _c(w)
    sdt = np.uint8 if dtype == "mxfp4" else np.float32
    s = _c(s, sdt)
    E, K, N = w.shape
    out = ctypes.c_double()
    _check(lib().orc_weight_value(_ptr(w), _ptr(s), _DT[dtype], e, K, N, k, n, ctypes.byref(out)), "weight_value")
    return out.value


def e4m3_encode(v):
    """E4M3 codes (uint8) of fp32 values v: round to nearest even, magnitudes
    of 448 and above saturating to 448."""
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    _check(lib().orc_e4m3_encode(_ptr(v), v.size, _ptr(out)), "e4m3_encode")
    return out


def quant_rows_e4m3(x):
    """Per-row E4M3 quantisation of activations x [T][m] (fp32, or bf16 as
    uint16): (values in double, codes, fp32 scales)."""
    x = _c(x)
    T, m = x.shape
    out = np.empty((T, m), np.float64)
    codes = np.empty((T, m), np.uint8)
    scales = np.empty(T, np.float32)
    _check(lib().orc_quant_rows_e4m3(_ptr(x), _xdt(x), T, m, _ptr(out), _ptr(codes), _ptr(scales)),
           "quant_rows_e4m3")
    return out, codes, scales


def quant_rows_i8(x):
    """Per-row int8 quantisation of activations x [T][m] (fp32, or bf16 as
    uint16): (values in double, int8 codes, fp32 scales)."""
    x = _c(x)
    T, m = x.shape
    out = np.empty((T, m), np.float64)
    codes = np.empty((T, m), np.int8)
    scales = np.empty(T, np.float32)
    _check(lib().orc_quant_rows_i8(_ptr(x), _xdt(x), T, m, _ptr(out), _ptr(codes), _ptr(scales)), "quant_rows_i8")
    return out, codes, scales


def router_logits(x, wg, bias=None):
    x = _c(x)
    wg = _c(wg, np.float32)
    bias = _c(bias, np.float32)
    T, m = x.shape
    E = wg.shape[1]
    out = np.empty((T, E), np.float32)
    _check(lib().orc_router_logits(_ptr(x), _xdt(x), _ptr(wg), _ptr(bias), T, m, E, _ptr(out)), "router")
    return out


NORM_LAYER, NORM_RMS = 1, 2


def norm(x, kind, gamma, beta=None, eps=1e-5):
    """Layer norm (NORM_LAYER) or RMS norm (NORM_RMS) of each row, in double."""
    x = _c(x)
    gamma = _c(gamma, np.float32)
    beta = _c(beta, np.float32)
    T, m = x.shape
    out = np.empty((T, m), np.float64)
    _check(lib().orc_norm(_ptr(x), _xdt(x), T, m, kind, _ptr(gamma), _ptr(beta), float(eps), _ptr(out)), "norm")
    return out


def topk(logits, k):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _check(lib().orc_topk(_ptr(logits), T, E, k, _ptr(idx), _ptr(w)), "topk")
    return idx, w


def dispatch(idx, E):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv = np.empty(T * k, np.int32)
    _check(lib().orc_dispatch(_ptr(idx), T, E, k, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv)), "dispatch")
    return counts, offsets, perm, inv


def expert_apply(X: Experts, e, xrow):
    """One expert on one activation row (float64); returns (o, ops[3])."""
    xrow = _c(xrow, np.float64)
    o = np.empty(X.m, np.float64)
    ops = np.zeros(3, np.uint64)
    _check(lib().orc_expert_apply(ctypes.byref(X._s), e, _ptr(xrow), _ptr(o), _ptr(ops)), "expert_apply")
    return o, ops


def expert_rows(X: Experts, x, k, perm, offsets, rows=None):
    """Unweighted expert outputs for permuted rows (all T*k when rows is None)."""
    x = _c(x)
    perm = _c(perm, np.int32)
    offsets = _c(offsets, np.int32)
    rows = _c(rows, np.int32)
    T = x.shape[0]
    n = T * k if rows is None else len(rows)
    out = np.empty((n, X.m), np.float64)
    ops = np.zeros(3, np.uint64)
    _check(lib().orc_expert_rows(ctypes.byref(X._s), _ptr(x), _xdt(x), T, k, _ptr(perm), _ptr(offsets),
                                 _ptr(rows), n, _ptr(out), _ptr(ops)), "expert_rows")
    return out, ops


def combine(y_perm, inv_perm, idx, w):
    y_perm = _c(y_perm, np.float64)
    inv_perm = _c(inv_perm, np.int32)
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    T, k = idx.shape
    m = y_perm.shape[1]
    y = np.empty((T, m), np.float64)
    _check(lib().orc_combine(_ptr(y_perm), _ptr(inv_perm), _ptr(idx), _ptr(w), T, m, k, _ptr(y)), "combine")
    return y


def forward_tokens(X: Experts, x, wg, bias, k, tokens, logits=None):
    """End-to-end output rows for the given tokens; returns (y, idx, w, ops)."""
    x = _c(x)
    wg = _c(wg, np.float32)
    bias = _c(bias, np.float32)
    logits = _c(logits, np.float32)
    tokens = _c(np.asarray(tokens), np.int32)
    T = x.shape[0]
    n = len(tokens)
    y = np.empty((n, X.m), np.float64)
    idx = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float32)
    ops = np.zeros(3, np.uint64)
    _check(lib().orc_forward_tokens(ctypes.byref(X._s), _ptr(x), _xdt(x), _ptr(wg), _ptr(bias), _ptr(logits),
                                    T, k, _ptr(tokens), n, _ptr(y), _ptr(idx), _ptr(w), _ptr(ops)),
           "forward_tokens")
    return y, idx, w, ops


def dense_masked(X: Experts, x, idx, w):
    x = _c(x)
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    T, k = idx.shape
    y = np.empty((T, X.m), np.float64)
    _check(lib().orc_dense_masked(ctypes.byref(X._s), _ptr(x), _xdt(x), _ptr(idx), _ptr(w), T, k, _ptr(y)),
           "dense_masked")
    return y


def layer_forward(X: Experts, x, wg, bias, k, logits=None):
    """Whole layer through the routed path: returns a dict of every stage."""
    if logits is None:
        logits = router_logits(x, wg, bias)
    idx, w = topk(logits, k)
    counts, offsets, perm, inv = dispatch(idx, X.E)
    y_perm, ops = expert_rows(X, x, k, perm, offsets)
    y = combine(y_perm, inv, idx, w)
    return dict(logits=logits, idx=idx, w=w, counts=counts, offsets=offsets, perm=perm, inv_perm=inv,
                y_perm=y_perm, y=y, ops=ops)
