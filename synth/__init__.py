"""Seeded synthetic MoE layers, shared input source for the oracle and the GPU path.

Nothing here computes any part of the MoE layer: it only draws activations,
router weights and expert weights (and quantises the int8 ones), in the
canonical row-major layouts the C ABI and the oracle both take:

    x      [T][m]      fp32, or bf16 stored as uint16 bit patterns
    wg     [m][E]      fp32 router weights
    bias   [E] fp32 or None (router logit bias, only for the skewed layer)
    w1     [E][m][p]   first projection (ReLU MLP) or gate projection (SwiGLU)
    w3     [E][m][p]   up projection (SwiGLU only) or None
    w2     [E][p][m]   second / down projection
    s1, s3 [E][p], s2 [E][m]   fp32 per-output-channel scales (int8, int4, fp8)
    s1, s3 [E][m/32][p], s2 [E][p/32][m]   uint8 E8M0 block scales (MXFP4)

The generator is SplitMix64 in counter form with Box-Muller normals; see
synth/gen.c.  Tensor stream ids: x=0, wg=1, w1=3, w3=4, w2=5.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libmoe_synth.so")

TID_X, TID_WG, TID_BIAS, TID_W1, TID_W3, TID_W2 = 0, 1, 2, 3, 4, 5


def build() -> str:
    """Compile the generator with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(
        ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"],
        check=True,
    )
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64, u32, i64, dbl = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        L.synth_splitmix64_at.argtypes = [u64, u64]
        L.synth_splitmix64_at.restype = u64
        L.synth_normal_at.argtypes = [u64, u64]
        L.synth_normal_at.restype = dbl
        L.synth_f32_to_bf16.argtypes = [ctypes.c_float]
        L.synth_f32_to_bf16.restype = ctypes.c_uint16
        L.synth_fill_normal_f32.argtypes = [u64, u32, dbl, i64, vp]
        L.synth_fill_normal_f32.restype = None
        L.synth_fill_normal_bf16.argtypes = [u64, u32, dbl, i64, vp]
        L.synth_fill_normal_bf16.restype = None
        L.synth_fill_int8_quant.argtypes = [u64, u32, dbl, i64, i64, i64, vp, vp]
        L.synth_fill_int8_quant.restype = ctypes.c_int
        L.synth_fill_intq_quant.argtypes = [u64, u32, dbl, i64, i64, i64, ctypes.c_int, vp, vp]
        L.synth_fill_intq_quant.restype = ctypes.c_int
        L.synth_fill_fp8_quant.argtypes = [u64, u32, dbl, i64, i64, i64, vp, vp]
        L.synth_fill_fp8_quant.restype = ctypes.c_int
        L.synth_fill_mxfp4_quant.argtypes = [u64, u32, dbl, i64, i64, i64, vp, vp]
        L.synth_fill_mxfp4_quant.restype = ctypes.c_int
        _lib = L
    return _lib


def normal_f32(seed: int, tid: int, sigma: float, shape) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    lib().synth_fill_normal_f32(seed, tid, sigma, out.size, out.ctypes.data)
    return out


def normal_bf16(seed: int, tid: int, sigma: float, shape) -> np.ndarray:
    """bf16 values as uint16 bit patterns."""
    out = np.empty(shape, dtype=np.uint16)
    lib().synth_fill_normal_bf16(seed, tid, sigma, out.size, out.ctypes.data)
    return out


def int8_quant(seed: int, tid: int, sigma: float, E: int, K: int, N: int):
    q = np.empty((E, K, N), dtype=np.int8)
    s = np.empty((E, N), dtype=np.float32)
    rc = lib().synth_fill_int8_quant(seed, tid, sigma, E, K, N, q.ctypes.data, s.ctypes.data)
    if rc != 0:
        raise MemoryError("synth_fill_int8_quant failed")
    return q, s


def int4_quant(seed: int, tid: int, sigma: float, E: int, K: int, N: int):
    """As int8_quant with q in [-7, 7] (held one per int8 byte)."""
    q = np.empty((E, K, N), dtype=np.int8)
    s = np.empty((E, N), dtype=np.float32)
    rc = lib().synth_fill_intq_quant(seed, tid, sigma, E, K, N, 7, q.ctypes.data, s.ctypes.data)
    if rc != 0:
        raise MemoryError("synth_fill_intq_quant failed")
    return q, s


def fp8_quant(seed: int, tid: int, sigma: float, E: int, K: int, N: int):
    """OCP E4M3 codes (uint8) with per-output-channel fp32 scales, the
    column's largest magnitude at 448."""
    q = np.empty((E, K, N), dtype=np.uint8)
    s = np.empty((E, N), dtype=np.float32)
    if lib().synth_fill_fp8_quant(seed, tid, sigma, E, K, N, q.ctypes.data, s.ctypes.data) != 0:
        raise MemoryError("synth_fill_fp8_quant failed")
    return q, s


def mxfp4_quant(seed: int, tid: int, sigma: float, E: int, K: int, N: int):
    """MXFP4: E2M1 codes (one per uint8) and one E8M0 exponent (uint8) per
    block of 32 consecutive k of a column, [E][K/32][N]."""
    q = np.empty((E, K, N), dtype=np.uint8)
    s = np.empty((E, K // 32, N), dtype=np.uint8)
    if lib().synth_fill_mxfp4_quant(seed, tid, sigma, E, K, N, q.ctypes.data, s.ctypes.data) != 0:
        raise MemoryError("synth_fill_mxfp4_quant failed")
    return q, s


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of uint16 bf16 bit patterns to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def zipf_logit_bias(E: int, s: float) -> np.ndarray:
    """b[e] = ln p_e with p_e = (e+1)^-s / sum_r r^-s: expert 0 is the hottest."""
    w = np.array([(e + 1) ** (-s) for e in range(E)], dtype=np.float64)
    return np.log(w / w.sum()).astype(np.float32)


@dataclass
class LayerSpec:
    name: str
    T: int
    m: int
    p: int
    E: int
    k: int
    kind: str  # "relu" | "swiglu"
    x_dtype: str  # "f32" | "bf16"
    w_dtype: str  # "f32" | "bf16" | "i8" | "i8a8" | "i4" | "fp8" | "fp8a8" | "mxfp4"
    seed: int
    sigma_x: float = 1.0
    sigma_router: float = 0.02
    sigma_w: float = 0.02
    zipf_s: float | None = None
    note: str = ""

    def expert_bytes(self) -> int:
        """|E| of one expert: (mp + pm) * dtype for the two-matrix MLP, 3*m*p*dtype for SwiGLU."""
        nmat = 2 if self.kind == "relu" else 3
        return int(nmat * self.m * self.p * {"f32": 4, "bf16": 2, "i8": 1, "i8a8": 1, "i4": 0.5, "fp8": 1, "fp8a8": 1,
                                             "mxfp4": 0.5 + 1 / 32}[self.w_dtype])


# The five measured layers.  Shapes follow Mixtral-8x7B (E=8, m=4096, p=14336)
# and Phi-3.5-MoE (E=16, p=6400) expert shapes as named in the GPU-cache
# article (MoE模型推理优化：GPU缓存与CPU协同计算实践, sections 1 and 5.1).
CONFIGS = {
    "c1": LayerSpec("tiny_relu_f32", 32, 256, 512, 8, 2, "relu", "f32", "f32", 0,
                    sigma_router=0.05, sigma_w=0.05,
                    note="tiny fp32 two-layer ReLU MLP experts"),
    "c2": LayerSpec("mixtral_decode_bf16", 16, 4096, 14336, 8, 2, "swiglu", "bf16", "bf16", 1,
                    note="Mixtral-8x7B-shaped decode, uniform routing"),
    "c3": LayerSpec("phi35_skewed_bf16", 256, 4096, 6400, 16, 2, "swiglu", "bf16", "bf16", 2,
                    zipf_s=1.2, note="Phi-3.5-MoE-shaped, Zipf(1.2) expert popularity"),
    "c4": LayerSpec("mixtral_prefill_bf16", 8192, 4096, 14336, 8, 2, "swiglu", "bf16", "bf16", 3,
                    note="Mixtral-8x7B-shaped prefill, uniform routing"),
    "c5": LayerSpec("mixtral_decode_int8", 64, 4096, 14336, 8, 2, "swiglu", "bf16", "i8", 4,
                    note="Mixtral-8x7B-shaped decode, int8 weights with per-channel fp32 scales"),
    # a next row (lower-precision weights): the int8 layer with int4 weights
    "c6": LayerSpec("mixtral_decode_int4", 64, 4096, 14336, 8, 2, "swiglu", "bf16", "i4", 5,
                    note="Mixtral-8x7B-shaped decode, int4 weights with per-channel fp32 scales"),
    # the integer weights at prefill size: the grouped GEMM with the dequant fused
    "c7": LayerSpec("mixtral_prefill_int8", 8192, 4096, 14336, 8, 2, "swiglu", "bf16", "i8", 6,
                    note="Mixtral-8x7B-shaped prefill, int8 weights with per-channel fp32 scales"),
    "c8": LayerSpec("mixtral_prefill_int4", 8192, 4096, 14336, 8, 2, "swiglu", "bf16", "i4", 7,
                    note="Mixtral-8x7B-shaped prefill, int4 weights with per-channel fp32 scales"),
    # 8-bit and 4-bit float weights (OCP E4M3 with per-channel scales; MXFP4)
    "c9": LayerSpec("mixtral_decode_fp8", 64, 4096, 14336, 8, 2, "swiglu", "bf16", "fp8", 8,
                    note="Mixtral-8x7B-shaped decode, E4M3 weights with per-channel fp32 scales"),
    "c10": LayerSpec("mixtral_decode_mxfp4", 64, 4096, 14336, 8, 2, "swiglu", "bf16", "mxfp4", 9,
                     note="Mixtral-8x7B-shaped decode, MXFP4 weights (E2M1, E8M0 scale per 32 k)"),
    "c11": LayerSpec("mixtral_prefill_fp8", 8192, 4096, 14336, 8, 2, "swiglu", "bf16", "fp8", 10,
                     note="Mixtral-8x7B-shaped prefill, E4M3 weights with per-channel fp32 scales"),
    # the same weights with each token's expert input quantised to E4M3 (one
    # scale per token): the first projection runs on the fp8 matrix cores
    "c12": LayerSpec("mixtral_prefill_fp8a8", 8192, 4096, 14336, 8, 2, "swiglu", "bf16", "fp8a8", 10,
                     note="Mixtral-8x7B-shaped prefill, E4M3 weights and per-token E4M3 activations"),
    "c13": LayerSpec("mixtral_decode_fp8a8", 64, 4096, 14336, 8, 2, "swiglu", "bf16", "fp8a8", 8,
                     note="Mixtral-8x7B-shaped decode, E4M3 weights and per-token E4M3 activations"),
    # int8 weights and int8 activations (the INT8 GeMM with both operands
    # quantised): the first projection on the int8 matrix cores
    "c14": LayerSpec("mixtral_prefill_i8a8", 8192, 4096, 14336, 8, 2, "swiglu", "bf16", "i8a8", 6,
                     note="Mixtral-8x7B-shaped prefill, int8 weights and per-token int8 activations"),
    # MXFP4 weights at prefill size: the grouped GEMM on the weights expanded
    # to bf16
    "c15": LayerSpec("mixtral_prefill_mxfp4", 8192, 4096, 14336, 8, 2, "swiglu", "bf16", "mxfp4", 11,
                     note="Mixtral-8x7B-shaped prefill, MXFP4 weights (E2M1, E8M0 scale per 32 k)"),
}


def spec(name_or_spec) -> LayerSpec:
    if isinstance(name_or_spec, LayerSpec):
        return name_or_spec
    if name_or_spec in CONFIGS:
        return CONFIGS[name_or_spec]
    for s in CONFIGS.values():
        if s.name == name_or_spec:
            return s
    raise KeyError(name_or_spec)


def make_layer(sp: LayerSpec, with_x: bool = True, with_weights: bool = True) -> dict:
    """Draw the layer's tensors.  Returns a dict of numpy arrays (see module doc)."""
    T, m, p, E = sp.T, sp.m, sp.p, sp.E
    out = {"spec": sp}
    if with_x:
        if sp.x_dtype == "f32":
            out["x"] = normal_f32(sp.seed, TID_X, sp.sigma_x, (T, m))
        else:
            out["x"] = normal_bf16(sp.seed, TID_X, sp.sigma_x, (T, m))
    out["wg"] = normal_f32(sp.seed, TID_WG, sp.sigma_router, (m, E))
    out["bias"] = zipf_logit_bias(E, sp.zipf_s) if sp.zipf_s is not None else None
    out["w1"] = out["w3"] = out["w2"] = None
    out["s1"] = out["s3"] = out["s2"] = None
    if with_weights:
        mats = [("w1", TID_W1, (E, m, p)), ("w2", TID_W2, (E, p, m))]
        if sp.kind == "swiglu":
            mats.insert(1, ("w3", TID_W3, (E, m, p)))
        for key, tid, shape in mats:
            if sp.w_dtype == "f32":
                out[key] = normal_f32(sp.seed, tid, sp.sigma_w, shape)
            elif sp.w_dtype == "bf16":
                out[key] = normal_bf16(sp.seed, tid, sp.sigma_w, shape)
            else:
                quant = {"i8": int8_quant, "i8a8": int8_quant, "i4": int4_quant, "fp8": fp8_quant, "fp8a8": fp8_quant,
                         "mxfp4": mxfp4_quant}[sp.w_dtype]
                q, s = quant(sp.seed, tid, sp.sigma_w, *shape)
                out[key] = q
                out["s" + key[1:]] = s
    return out
