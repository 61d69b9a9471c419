"""CPU oracle for blockwise NF4/FP4 quantization and the 4-bit x bf16 product.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may load it; the product library never does.

A thin numpy wrapper over ``nf4_oracle.c`` (plain C, built with gcc, no SIMD
intrinsics, no BLAS). bf16 arrays are carried as ``numpy.uint16`` bit patterns.
Every function states which passage of the pages it follows; see the C file's
header for the sources and the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnf4_oracle.so")

NF4 = 0
FP4 = 1
QUANT_TYPES = {"nf4": NF4, "fp4": FP4}

_lib = None


def ensure_built(force: bool = True) -> str:
    """Compile nf4_oracle.c with gcc into libnf4_oracle.so (IEEE binary32, no
    contraction, no fast-math); with force=False only when the library is
    missing or older than the source. (Not named `build`: importing the
    submodule oracle.build would replace that attribute of the package.)"""
    from oracle.build import build_oracle

    return build_oracle(force=force)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        ensure_built(force=False)
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int
    lib.orc_norm_ppf.restype = ctypes.c_double
    lib.orc_norm_ppf.argtypes = [ctypes.c_double]
    lib.orc_codebook.restype = i32
    lib.orc_codebook.argtypes = [i32, P]
    lib.orc_nearest_code.restype = i32
    lib.orc_nearest_code.argtypes = [i32, ctypes.c_float]
    lib.orc_f32_to_bf16.restype = ctypes.c_uint16
    lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.orc_quantize.restype = i32
    lib.orc_quantize.argtypes = [P, i64, i32, i32, P, P]
    lib.orc_double_quant.restype = i32
    lib.orc_double_quant.argtypes = [P, i64, i32, P, P]
    lib.orc_dequantize.restype = i32
    lib.orc_dequantize.argtypes = [P, i64, i32, i32, P, P, P, i32, P, P]
    lib.orc_matmul_bf16.restype = i32
    lib.orc_matmul_bf16.argtypes = [P, P, i64, i64, i64, P]
    lib.orc_matmul_bf16_sampled.restype = i32
    lib.orc_matmul_bf16_sampled.argtypes = [P, P, i64, P, P, i64, P]
    lib.orc_gemv_quantized.restype = i32
    lib.orc_gemv_quantized.argtypes = [P, i64, P, i64, i64, i32, i32, P, P, P, i32, P]
    lib.orc_quantize_typed.restype = i32
    lib.orc_quantize_typed.argtypes = [P, i32, i64, i32, i32, P, P]
    lib.orc_double_quant_centred.restype = i32
    lib.orc_double_quant_centred.argtypes = [P, i64, i32, P, P, P]
    lib.orc_dequantize_typed.restype = i32
    lib.orc_dequantize_typed.argtypes = [P, i64, i32, i32, P, P, P, P, i32, P, P, P]
    lib.orc_matmul_typed.restype = i32
    lib.orc_matmul_typed.argtypes = [P, P, i32, i64, i64, i64, P]
    lib.orc_gemv_quantized_typed.restype = i32
    lib.orc_gemv_quantized_typed.argtypes = [P, i32, i64, P, i64, i64, i32, i32, P, P, P, P, i32, P]
    lib.orc_gemv_quantized_threads.restype = i32
    lib.orc_gemv_quantized_threads.argtypes = [P, i32, i64, P, i64, i64, i32, i32, P, P, P, P, i32, P,
                                               i32, i64]
    lib.orc_convert.restype = i32
    lib.orc_convert.argtypes = [P, i32, i64, P, i32]
    lib.orc_f32_to_f16.restype = ctypes.c_uint16
    lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
    lib.orc_f16_to_f32.restype = ctypes.c_float
    lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
    _lib = lib
    return lib


def _qt(quant_type) -> int:
    if isinstance(quant_type, str):
        return QUANT_TYPES[quant_type]
    return int(quant_type)


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def norm_ppf(p: float) -> float:
    """Standard normal quantile, bisection on the C library's erfc."""
    return _load().orc_norm_ppf(float(p))


def codebook(quant_type="nf4") -> np.ndarray:
    """fp32[16] code values indexed by the 4-bit code (NF4 page, table
    数学原理对比 row 数值表示; FP4 per the page's closing notes)."""
    out = np.zeros(16, dtype=np.float32)
    _check(_load().orc_codebook(_qt(quant_type), _ptr(out)), "codebook")
    return out


def nearest_code(s: float, quant_type="nf4") -> int:
    """Code of the codebook value nearest to the fp32 value s (ties to the
    smaller value)."""
    return int(_load().orc_nearest_code(_qt(quant_type), ctypes.c_float(float(s))))


def f32_to_bf16(f: float) -> int:
    return int(_load().orc_f32_to_bf16(ctypes.c_float(float(f))))


def num_blocks(n: int, bs: int) -> int:
    return (n + bs - 1) // bs


def quantize(w_bf16: np.ndarray, blocksize: int = 64, quant_type="nf4"):
    """Blockwise quantize a flattened bf16 tensor. Returns (packed uint8[ceil(n/2)],
    absmax float32[ceil(n/bs)])."""
    w = np.ascontiguousarray(w_bf16.reshape(-1), dtype=np.uint16)
    n = w.size
    packed = np.zeros((n + 1) // 2, dtype=np.uint8)
    absmax = np.zeros(num_blocks(n, blocksize), dtype=np.float32)
    _check(_load().orc_quantize(_ptr(w), n, blocksize, _qt(quant_type), _ptr(packed), _ptr(absmax)),
           "quantize")
    return packed, absmax


def double_quant(absmax: np.ndarray, blocksize2: int = 256):
    """Quantize fp32 block scales to int8 with one fp32 scale per group.
    Returns (q int8[nb], s2 float32[ceil(nb/bs2)])."""
    a = np.ascontiguousarray(absmax.reshape(-1), dtype=np.float32)
    nb = a.size
    q = np.zeros(nb, dtype=np.int8)
    s2 = np.zeros(num_blocks(nb, blocksize2), dtype=np.float32)
    _check(_load().orc_double_quant(_ptr(a), nb, blocksize2, _ptr(q), _ptr(s2)), "double_quant")
    return q, s2


def dequantize(packed: np.ndarray, n: int, blocksize: int = 64, quant_type="nf4", absmax=None,
               absmax_q=None, absmax_scale=None, blocksize2: int = 256, absmax_offset=None,
               half: str = "bf16"):
    """Dequantize. Returns (fp32[n], 16-bit bit patterns uint16[n]) where the
    16-bit output is the bf16 (half="bf16") or fp16 (half="fp16") rounding of
    the fp32 value. absmax_offset: the group offsets of the mean-centred
    double quant (with absmax_q / absmax_scale)."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    out32 = np.zeros(n, dtype=np.float32)
    out16 = np.zeros(n, dtype=np.uint16)
    a = None if absmax is None else np.ascontiguousarray(absmax, dtype=np.float32)
    q = None if absmax_q is None else np.ascontiguousarray(absmax_q, dtype=np.int8)
    s2 = None if absmax_scale is None else np.ascontiguousarray(absmax_scale, dtype=np.float32)
    off = None if absmax_offset is None else np.ascontiguousarray(absmax_offset, dtype=np.float32)
    if half not in ("bf16", "fp16"):
        raise ValueError(half)
    _check(_load().orc_dequantize_typed(
        _ptr(p), n, blocksize, _qt(quant_type), _ptr(a), _ptr(q), _ptr(s2), _ptr(off), blocksize2,
        _ptr(out32), _ptr(out16) if half == "bf16" else None,
        _ptr(out16) if half == "fp16" else None), "dequantize")
    return out32, out16


def matmul_bf16(x_bf16: np.ndarray, wc_bf16: np.ndarray) -> np.ndarray:
    """fp64 y = x @ Wc^T for bf16 x [M, K] and bf16 Wc [N, K]."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    w = np.ascontiguousarray(wc_bf16, dtype=np.uint16)
    M, K = x.shape
    N, K2 = w.shape
    assert K == K2
    y = np.zeros((M, N), dtype=np.float64)
    _check(_load().orc_matmul_bf16(_ptr(x), _ptr(w), M, N, K, _ptr(y)), "matmul")
    return y


def linear_bf16(x_bf16: np.ndarray, wc_bf16: np.ndarray, bias_bf16: np.ndarray | None = None):
    """fp64 y = x @ Wc^T + bias for bf16 x [M, K], Wc [N, K] and bias [N] (or no
    bias): a linear layer whose bias is part of the product (repo page
    ossradar.top bitsandbytes, release notes 0.50.0, "Highlights": the fused
    4-bit kernels take the bias too). The bf16 bias is widened exactly."""
    y = matmul_bf16(x_bf16, wc_bf16)
    if bias_bf16 is not None:
        b = np.ascontiguousarray(bias_bf16, dtype=np.uint16).astype(np.uint32) << 16
        y = y + b.view(np.float32).astype(np.float64)[None, :]
    return y


def matmul_bf16_sampled(x_bf16: np.ndarray, wc_bf16: np.ndarray, ms, ns) -> np.ndarray:
    """fp64 y[i] = sum_k Wc[ns[i], k] * x[ms[i], k] for the listed positions."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    w = np.ascontiguousarray(wc_bf16, dtype=np.uint16)
    K = x.shape[1]
    assert w.shape[1] == K
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    assert ms.size == ns.size
    assert ms.size == 0 or (ms.min() >= 0 and ms.max() < x.shape[0] and ns.min() >= 0
                            and ns.max() < w.shape[0])
    y = np.zeros(ms.size, dtype=np.float64)
    _check(_load().orc_matmul_bf16_sampled(_ptr(x), _ptr(w), K, _ptr(ms), _ptr(ns), ms.size, _ptr(y)),
           "matmul_sampled")
    return y


def gemv_quantized(x_bf16: np.ndarray, packed: np.ndarray, N: int, K: int, blocksize: int = 64,
                   quant_type="nf4", absmax=None, absmax_q=None, absmax_scale=None,
                   blocksize2: int = 256) -> np.ndarray:
    """fp64 y [M, N] = x @ bf16(dequant(W))^T, dequantizing row by row."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    M = x.shape[0]
    assert x.shape[1] == K
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    a = None if absmax is None else np.ascontiguousarray(absmax, dtype=np.float32)
    q = None if absmax_q is None else np.ascontiguousarray(absmax_q, dtype=np.int8)
    s2 = None if absmax_scale is None else np.ascontiguousarray(absmax_scale, dtype=np.float32)
    y = np.zeros((M, N), dtype=np.float64)
    _check(_load().orc_gemv_quantized(_ptr(x), M, _ptr(p), N, K, blocksize, _qt(quant_type), _ptr(a),
                                      _ptr(q), _ptr(s2), blocksize2, _ptr(y)), "gemv")
    return y


# ------------------------------------------------------------ element types

DTYPES = {"bf16": 0, "fp32": 1, "fp16": 2}


def _dt(dtype) -> int:
    return DTYPES[dtype] if isinstance(dtype, str) else int(dtype)


def _typed(a: np.ndarray, dtype) -> np.ndarray:
    """bf16 / fp16 tensors as uint16 bit patterns, fp32 as float32."""
    if _dt(dtype) == DTYPES["fp32"]:
        return np.ascontiguousarray(a, dtype=np.float32)
    return np.ascontiguousarray(a, dtype=np.uint16)


def convert(a: np.ndarray, src, dst) -> np.ndarray:
    """Elementwise conversion between bf16 / fp16 (uint16 bits) and fp32
    (float32), through the exact fp32 value, rounding to nearest even."""
    x = _typed(a, src).reshape(-1)
    out = np.zeros(x.size, dtype=np.float32 if _dt(dst) == DTYPES["fp32"] else np.uint16)
    _check(_load().orc_convert(_ptr(x), _dt(src), x.size, _ptr(out), _dt(dst)), "convert")
    return out.reshape(np.shape(a))


def quantize_typed(w: np.ndarray, dtype="bf16", blocksize: int = 64, quant_type="nf4"):
    """Blockwise quantize a flattened tensor of bf16 / fp16 (uint16 bits) or
    fp32 values, each taken as its exact fp32 value. Returns (packed, absmax)."""
    x = _typed(w, dtype).reshape(-1)
    n = x.size
    packed = np.zeros((n + 1) // 2, dtype=np.uint8)
    absmax = np.zeros(num_blocks(n, blocksize), dtype=np.float32)
    _check(_load().orc_quantize_typed(_ptr(x), _dt(dtype), n, blocksize, _qt(quant_type),
                                      _ptr(packed), _ptr(absmax)), "quantize_typed")
    return packed, absmax


def double_quant_centred(absmax: np.ndarray, blocksize2: int = 256):
    """Mean-centred second level: per group of bs2 scales, mu = pairwise fp32
    sum / count, s2 = RN(max |a - mu| / 127), q = clamp(rint((a - mu) / s2)).
    Returns (q int8[nb], s2 float32[ng], mu float32[ng])."""
    a = np.ascontiguousarray(absmax.reshape(-1), dtype=np.float32)
    nb = a.size
    q = np.zeros(nb, dtype=np.int8)
    ng = num_blocks(nb, blocksize2)
    s2 = np.zeros(ng, dtype=np.float32)
    mu = np.zeros(ng, dtype=np.float32)
    _check(_load().orc_double_quant_centred(_ptr(a), nb, blocksize2, _ptr(q), _ptr(s2), _ptr(mu)),
           "double_quant_centred")
    return q, s2, mu


def matmul_typed(x: np.ndarray, wc: np.ndarray, dtype="bf16") -> np.ndarray:
    """fp64 y = x @ Wc^T for x [M, K] and Wc [N, K] of one compute dtype."""
    xx = _typed(x, dtype)
    ww = _typed(wc, dtype)
    M, K = xx.shape
    N, K2 = ww.shape
    assert K == K2
    y = np.zeros((M, N), dtype=np.float64)
    _check(_load().orc_matmul_typed(_ptr(xx), _ptr(ww), _dt(dtype), M, N, K, _ptr(y)), "matmul")
    return y


def gemv_quantized_typed(x: np.ndarray, packed: np.ndarray, N: int, K: int, blocksize: int = 64,
                         quant_type="nf4", absmax=None, absmax_q=None, absmax_scale=None,
                         absmax_offset=None, blocksize2: int = 256, dtype="bf16") -> np.ndarray:
    """fp64 y [M, N] = x @ dtype(dequant(W))^T in the compute dtype `dtype`."""
    xx = _typed(x, dtype)
    if xx.ndim == 1:
        xx = xx.reshape(1, -1)
    M = xx.shape[0]
    assert xx.shape[1] == K
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    a = None if absmax is None else np.ascontiguousarray(absmax, dtype=np.float32)
    q = None if absmax_q is None else np.ascontiguousarray(absmax_q, dtype=np.int8)
    s2 = None if absmax_scale is None else np.ascontiguousarray(absmax_scale, dtype=np.float32)
    off = None if absmax_offset is None else np.ascontiguousarray(absmax_offset, dtype=np.float32)
    y = np.zeros((M, N), dtype=np.float64)
    _check(_load().orc_gemv_quantized_typed(_ptr(xx), _dt(dtype), M, _ptr(p), N, K, blocksize,
                                            _qt(quant_type), _ptr(a), _ptr(q), _ptr(s2), _ptr(off),
                                            blocksize2, _ptr(y)), "gemv_typed")
    return y


def gemv_quantized_threads(x: np.ndarray, packed: np.ndarray, N: int, K: int, threads: int,
                           blocksize: int = 64, quant_type="nf4", absmax=None, absmax_q=None,
                           absmax_scale=None, absmax_offset=None, blocksize2: int = 256,
                           dtype="bf16") -> np.ndarray:
    """gemv_quantized_typed split over `threads` host threads by rows (whole
    double-quant groups per thread); bitwise the single-threaded result."""
    xx = _typed(x, dtype)
    if xx.ndim == 1:
        xx = xx.reshape(1, -1)
    M = xx.shape[0]
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    a = None if absmax is None else np.ascontiguousarray(absmax, dtype=np.float32)
    q = None if absmax_q is None else np.ascontiguousarray(absmax_q, dtype=np.int8)
    s2 = None if absmax_scale is None else np.ascontiguousarray(absmax_scale, dtype=np.float32)
    off = None if absmax_offset is None else np.ascontiguousarray(absmax_offset, dtype=np.float32)
    # rows per share: whole groups of bs2 blocks
    import math
    row_blocks = K // blocksize
    align = blocksize2 // math.gcd(blocksize2, row_blocks) if q is not None else 1
    y = np.zeros((M, N), dtype=np.float64)
    _check(_load().orc_gemv_quantized_threads(
        _ptr(xx), _dt(dtype), M, _ptr(p), N, K, blocksize, _qt(quant_type), _ptr(a), _ptr(q),
        _ptr(s2), _ptr(off), blocksize2, _ptr(y), int(threads), align), "gemv_threads")
    return y
