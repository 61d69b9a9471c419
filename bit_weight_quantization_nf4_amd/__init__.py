"""Python binding of libnf4 (MI355X / gfx950): blockwise NF4/FP4 4-bit weight
quantization, double quantization, dequantization and the 4-bit x bf16 products.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in ``include/nf4.h``; PyTorch supplies device memory and the current
stream. There is no fallback: if ``libnf4.so`` is not built, importing the
low-level handle raises.

Functions mirror the C entry points: ``quantize`` (nf4_quantize /
nf4_quantize_ex), ``double_quant``, ``dequantize``, ``gemv``, ``gemm``,
``linear`` (nf4_linear / nf4_linear_ex), the grouped forms, plus ``codebook``
(host) and the size helpers. A quantized tensor is described by
:class:`QuantState`, the counterpart of the pages' 4-bit configuration
(quant_type, use_double_quant, compute dtype) plus the blocksizes.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnf4.so")

NF4_OK = 0
NF4_ERR_INVALID_ARGUMENT = 1
NF4_ERR_UNSUPPORTED = 2
NF4_ERR_MISALIGNED = 3
NF4_ERR_DEVICE = 4

QUANT_NF4 = 0
QUANT_FP4 = 1
DTYPE_BF16 = 0
DTYPE_FP32 = 1
DTYPE_FP16 = 2
DQ_NONE = 0
DQ_SYMMETRIC = 1
DQ_CENTRED = 2
ABI_VERSION = 3
GEMV_MAX_M = 64

_QT = {"nf4": QUANT_NF4, "fp4": QUANT_FP4}
_DT = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_FP32, torch.float16: DTYPE_FP16}


def _dq(mode) -> int:
    """Double-quant mode: False / 0 none, True / 1 / "symmetric", 2 / "centred"."""
    if isinstance(mode, str):
        return {"none": DQ_NONE, "symmetric": DQ_SYMMETRIC, "centred": DQ_CENTRED}[mode]
    return int(mode)


class QWeightDesc(ctypes.Structure):
    """ctypes mirror of ``nf4_qweight``."""

    _fields_ = [
        ("packed", ctypes.c_void_p),
        ("absmax", ctypes.c_void_p),
        ("absmax_q", ctypes.c_void_p),
        ("absmax_scale", ctypes.c_void_p),
        ("n", ctypes.c_int64),
        ("blocksize", ctypes.c_int32),
        ("quant_type", ctypes.c_int32),
        ("double_quant", ctypes.c_int32),
        ("blocksize2", ctypes.c_int32),
        ("absmax_offset", ctypes.c_void_p),
    ]


# (name, restype, argtypes) of every exported entry point
_P = ctypes.c_void_p
_SIGNATURES = [
    ("nf4_abi_version", ctypes.c_int32, []),
    ("nf4_status_string", ctypes.c_char_p, [ctypes.c_int32]),
    ("nf4_packed_bytes", ctypes.c_int64, [ctypes.c_int64]),
    ("nf4_num_blocks", ctypes.c_int64, [ctypes.c_int64, ctypes.c_int32]),
    ("nf4_codebook", ctypes.c_int32, [ctypes.c_int32, _P]),
    ("nf4_device_check", ctypes.c_int32, []),
    ("nf4_quantize", ctypes.c_int32,
     [_P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P]),
    ("nf4_quantize_grouped", ctypes.c_int32,
     [ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_int64),
      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p),
      ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
      ctypes.POINTER(ctypes.c_void_p), _P]),
    ("nf4_quantize_ex", ctypes.c_int32,
     [_P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
      ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P, _P]),
    ("nf4_double_quant", ctypes.c_int32, [_P, ctypes.c_int64, ctypes.c_int32, _P, _P, _P]),
    ("nf4_double_quant_ex", ctypes.c_int32,
     [_P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P]),
    ("nf4_dequantize", ctypes.c_int32, [ctypes.POINTER(QWeightDesc), ctypes.c_int32, _P, _P]),
    ("nf4_dequantize_grouped", ctypes.c_int32,
     [ctypes.c_int32, ctypes.POINTER(QWeightDesc), ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p),
      _P]),
    ("nf4_gemv", ctypes.c_int32,
     [_P, ctypes.c_int32, ctypes.POINTER(QWeightDesc), ctypes.c_int32, ctypes.c_int32,
      ctypes.c_int32, ctypes.c_int32, _P, _P]),
    ("nf4_gemv_grouped", ctypes.c_int32,
     [ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32, ctypes.POINTER(QWeightDesc),
      ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
      ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p), _P]),
    ("nf4_gemm", ctypes.c_int32,
     [_P, ctypes.c_int32, ctypes.POINTER(QWeightDesc), ctypes.c_int32, ctypes.c_int32,
      ctypes.c_int32, ctypes.c_int32, _P, _P]),
    ("nf4_linear", ctypes.c_int32,
     [_P, ctypes.c_int32, ctypes.POINTER(QWeightDesc), ctypes.c_int32, ctypes.c_int32, _P,
      ctypes.c_int32, ctypes.c_int32, _P, _P]),
    ("nf4_linear_ex", ctypes.c_int32,
     [_P, ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(QWeightDesc), ctypes.c_int32,
      ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int64, _P]),
    ("nf4_linear_workspace_bytes", ctypes.c_int64,
     [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
      ctypes.c_int32, ctypes.c_int32]),
    ("nf4_linear_ws", ctypes.c_int32,
     [_P, ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(QWeightDesc), ctypes.c_int32,
      ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int64, _P, ctypes.c_int64,
      _P]),
    ("nf4_linear_noalloc", ctypes.c_int32,
     [_P, ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(QWeightDesc), ctypes.c_int32,
      ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int64, _P]),
    ("nf4_gemv_grouped_ws", ctypes.c_int32,
     [ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32, ctypes.POINTER(QWeightDesc),
      ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
      ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p), _P, ctypes.c_int64, _P]),
]

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libnf4.so with typed entry points. Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libnf4.so not found at {LIB_PATH}: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    h = ctypes.CDLL(LIB_PATH)
    for name, res, args in _SIGNATURES:
        fn = getattr(h, name)
        fn.restype = res
        fn.argtypes = args
    if h.nf4_abi_version() != ABI_VERSION:
        raise RuntimeError("libnf4.so ABI version mismatch")
    _lib = h
    return h


def exported_names() -> list[str]:
    return [s[0] for s in _SIGNATURES]


class Nf4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().nf4_status_string(status).decode()}")


def _check(status: int, what: str) -> None:
    if status != NF4_OK:
        raise Nf4Error(status, what)


def _qt(quant_type) -> int:
    if isinstance(quant_type, str):
        return _QT[quant_type]
    return int(quant_type)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor) -> torch.Tensor:
    """Contiguous and 16-byte aligned (a copy only when a view is misaligned)."""
    t = t.contiguous()
    if t.data_ptr() % 16:
        t = t.clone()
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def packed_bytes(n: int) -> int:
    return int(lib().nf4_packed_bytes(n))


def num_blocks(n: int, blocksize: int) -> int:
    return int(lib().nf4_num_blocks(n, blocksize))


def codebook(quant_type="nf4") -> list[float]:
    """The 16 fp32 code values (host call), indexed by the 4-bit code."""
    buf = (ctypes.c_float * 16)()
    _check(lib().nf4_codebook(_qt(quant_type), ctypes.cast(buf, ctypes.c_void_p)), "nf4_codebook")
    return list(buf)


@dataclass
class QuantState:
    """A quantized tensor: packed codes plus block scales (device tensors).
    double_quant is the mode: 0 none, 1 symmetric, 2 mean-centred (True / False
    are accepted as 1 / 0)."""

    packed: torch.Tensor
    absmax: torch.Tensor
    absmax_q: torch.Tensor | None
    absmax_scale: torch.Tensor | None
    shape: tuple
    blocksize: int
    quant_type: str
    double_quant: int
    blocksize2: int = 256
    absmax_offset: torch.Tensor | None = None

    @property
    def n(self) -> int:
        n = 1
        for s in self.shape:
            n *= int(s)
        return n

    def desc(self) -> QWeightDesc:
        return QWeightDesc(
            _ptr(self.packed), _ptr(self.absmax), _ptr(self.absmax_q), _ptr(self.absmax_scale),
            self.n, self.blocksize, _QT[self.quant_type], _dq(self.double_quant), self.blocksize2,
            _ptr(self.absmax_offset))

    def nbytes(self) -> int:
        b = self.packed.numel()
        if _dq(self.double_quant):
            b += self.absmax_q.numel() + 4 * self.absmax_scale.numel()
            if self.absmax_offset is not None:
                b += 4 * self.absmax_offset.numel()
        else:
            b += 4 * self.absmax.numel()
        return b


def _new_state(shape, n: int, dev, blocksize: int, quant_type: str, mode: int) -> QuantState:
    nb = (n + blocksize - 1) // blocksize
    ng = (nb + 255) // 256
    return QuantState(torch.empty((n + 1) // 2, dtype=torch.uint8, device=dev),
                      torch.empty(nb, dtype=torch.float32, device=dev),
                      torch.empty(nb, dtype=torch.int8, device=dev) if mode else None,
                      torch.empty(ng, dtype=torch.float32, device=dev) if mode else None,
                      tuple(shape), blocksize, quant_type, mode, 256,
                      torch.empty(ng, dtype=torch.float32, device=dev)
                      if mode == DQ_CENTRED else None)


def _rows_view(w: torch.Tensor):
    """(tensor, rows, cols, ld): a row-strided 2-D view of w passed as is (unit
    element stride, any row stride), anything else as a contiguous copy."""
    es = w.element_size()
    if (w.dim() == 2 and w.stride(1) == 1 and w.stride(0) >= w.shape[1]
            and w.data_ptr() % 16 == 0 and (w.is_contiguous() or (
                w.shape[1] % 8 == 0 and (w.stride(0) * es) % 16 == 0))):
        return w, w.shape[0], w.shape[1], w.stride(0)
    w = _dev(w)
    return w, 1, w.numel(), w.numel()


def quantize(w: torch.Tensor, blocksize: int = 64, quant_type: str = "nf4",
             double_quant=False, out: QuantState | None = None) -> QuantState:
    """Quantize a bf16 / fp16 / fp32 device tensor (flattened row-major; a 2-D
    view with a row stride is read in place). nf4_quantize for contiguous bf16
    without the centred mode, nf4_quantize_ex otherwise. With ``out`` the
    result is written into its buffers instead of new ones."""
    if w.dtype not in _DT or not w.is_cuda:
        raise TypeError("quantize expects a bf16, fp16 or fp32 tensor on the GPU")
    mode = _dq(double_quant)
    if out is None:
        out = _new_state(w.shape, w.numel(), w.device, blocksize, quant_type, mode)
    if w.dtype == torch.bfloat16 and w.is_contiguous() and mode != DQ_CENTRED:
        w = _dev(w)
        _check(lib().nf4_quantize(_ptr(w), w.numel(), blocksize, _qt(quant_type), mode,
                                  _ptr(out.packed), _ptr(out.absmax), _ptr(out.absmax_q),
                                  _ptr(out.absmax_scale), _stream(w)), "nf4_quantize")
        return out
    src, rows, cols, ld = _rows_view(w)
    _check(lib().nf4_quantize_ex(_ptr(src), _DT[w.dtype], rows, cols, ld, blocksize,
                                 _qt(quant_type), mode, _ptr(out.packed), _ptr(out.absmax),
                                 _ptr(out.absmax_q), _ptr(out.absmax_scale),
                                 _ptr(out.absmax_offset), _stream(src)), "nf4_quantize_ex")
    return out


QUANT_MAX_GROUP = 16


def quantize_grouped(ws, blocksize: int = 64, quant_type: str = "nf4", double_quant=False,
                     outs=None):
    """nf4_quantize_grouped: several bf16 device tensors quantized in one call
    (one launch with double quant at blocksize 64/128/256). Returns their
    QuantStates (or fills ``outs``)."""
    count = len(ws)
    if count > QUANT_MAX_GROUP or (outs is not None and len(outs) != count):
        raise ValueError("quantize_grouped takes at most 16 tensors (and as many outs)")
    if count == 0:
        return []
    mode = _dq(double_quant)
    ws2, states = [], []
    for i, w in enumerate(ws):
        if w.dtype != torch.bfloat16 or not w.is_cuda:
            raise TypeError("quantize_grouped expects bf16 tensors on the GPU")
        w2 = _dev(w)
        ws2.append(w2)
        states.append(outs[i] if outs is not None else
                      _new_state(w2.shape, w2.numel(), w2.device, blocksize, quant_type, mode))
    vp = ctypes.c_void_p * count
    _check(lib().nf4_quantize_grouped(
        count, vp(*[_ptr(t) for t in ws2]), (ctypes.c_int64 * count)(*[t.numel() for t in ws2]),
        blocksize, _qt(quant_type), mode, vp(*[_ptr(q.packed) for q in states]),
        vp(*[_ptr(q.absmax) for q in states]), vp(*[_ptr(q.absmax_q) for q in states]),
        vp(*[_ptr(q.absmax_scale) for q in states]), _stream(ws2[0])), "nf4_quantize_grouped")
    return states


def double_quant(absmax: torch.Tensor, blocksize2: int = 256, mode=DQ_SYMMETRIC):
    """nf4_double_quant_ex: returns (absmax_q int8[nb], absmax_scale fp32[ng])
    and, in the centred mode, also absmax_offset fp32[ng]."""
    a = _dev(absmax)
    nb = a.numel()
    mode = _dq(mode)
    ng = (nb + blocksize2 - 1) // blocksize2
    q = torch.empty(nb, dtype=torch.int8, device=a.device)
    s2 = torch.empty(ng, dtype=torch.float32, device=a.device)
    mu = torch.empty(ng, dtype=torch.float32, device=a.device) if mode == DQ_CENTRED else None
    _check(lib().nf4_double_quant_ex(_ptr(a), nb, blocksize2, mode, _ptr(q), _ptr(s2), _ptr(mu),
                                     _stream(a)), "nf4_double_quant_ex")
    return (q, s2) if mode != DQ_CENTRED else (q, s2, mu)


def dequantize(qs: QuantState, out_dtype=torch.bfloat16, out: torch.Tensor | None = None):
    """nf4_dequantize to bf16 / fp16 (compute dtypes) or fp32, shaped like the source."""
    if out is None:
        out = torch.empty(qs.shape, dtype=out_dtype, device=qs.packed.device)
    d = qs.desc()
    _check(lib().nf4_dequantize(ctypes.byref(d), _DT[out.dtype], _ptr(out), _stream(qs.packed)),
           "nf4_dequantize")
    return out


def dequantize_grouped(qss, out_dtype=torch.bfloat16, outs=None):
    """nf4_dequantize_grouped: several quantized tensors dequantized in one
    launch; returns the list of outputs (or fills ``outs``)."""
    count = len(qss)
    if count > QUANT_MAX_GROUP or (outs is not None and len(outs) != count):
        raise ValueError("dequantize_grouped takes at most 16 tensors (and as many outs)")
    if count == 0:
        return []
    ys = [outs[i] if outs is not None else torch.empty(qs.shape, dtype=out_dtype,
                                                        device=qs.packed.device)
          for i, qs in enumerate(qss)]
    _check(lib().nf4_dequantize_grouped(count, (QWeightDesc * count)(*[q.desc() for q in qss]),
                                        _DT[ys[0].dtype],
                                        (ctypes.c_void_p * count)(*[_ptr(y) for y in ys]),
                                        _stream(qss[0].packed)), "nf4_dequantize_grouped")
    return ys


def _rows2d(t: torch.Tensor, cols: int):
    """(tensor, ld) for a [rows, cols] operand: a 2-D view with unit element
    stride is kept with its row stride, anything else flattened contiguously."""
    if t.dim() == 2 and t.shape[1] == cols and t.stride(1) == 1 and t.data_ptr() % 16 == 0 \
            and (t.shape[0] <= 1 or t.stride(0) >= cols):
        return t, (t.stride(0) if t.shape[0] > 1 else cols)
    t = _dev(t.reshape(-1, cols))
    return t, cols


def _product(fn, name, x, qs, out_dtype, out):
    if x.dtype not in _DT or not x.is_cuda:
        raise TypeError(f"{name} expects bf16 / fp16 / fp32 activations on the GPU")
    if len(qs.shape) != 2:
        raise ValueError(f"{name} expects a quantized [N, K] weight")
    N, K = (int(s) for s in qs.shape)
    x2 = _dev(x.reshape(-1, K))
    M = x2.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    d = qs.desc()
    _check(fn(_ptr(x2), M, ctypes.byref(d), N, K, _DT[x.dtype], _DT[out.dtype], _ptr(out),
              _stream(x2)), name)
    return out


def workspace_bytes(M: int, qs: QuantState, compute_dtype, out_dtype) -> int:
    """nf4_linear_workspace_bytes for x[M, K] . W^T with W = qs ([N, K])."""
    N, K = (int(s) for s in qs.shape)
    return int(lib().nf4_linear_workspace_bytes(M, N, K, qs.blocksize, _DT[compute_dtype],
                                                _DT[out_dtype], _dq(qs.double_quant)))


def _workspace(nbytes: int, device):
    """(pointer, bytes) of a fresh device workspace (torch's allocator, so it
    is safe under stream capture), or (None, 0)."""
    if nbytes <= 0:
        return None, 0, None
    t = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return t.data_ptr(), nbytes, t


def gemv(x: torch.Tensor, qs: QuantState, out_dtype=torch.float32, out=None,
         split: bool = True) -> torch.Tensor:
    """y[M, N] = x[M, K] . cd(W)^T for M <= 64; the compute dtype cd is x's
    dtype (bf16, fp16 or fp32). With split=True (nf4_gemv_grouped_ws) a
    product whose activations do not fit one compute unit's registers is split
    along K in a workspace this call allocates; split=False is nf4_gemv."""
    if not split:
        return _product(lib().nf4_gemv, "nf4_gemv", x, qs, out_dtype, out)
    return gemv_grouped([x], [qs], out_dtype, None if out is None else [out], split=True)[0]


GEMV_MAX_GROUP = 16


def gemv_grouped(xs, qss, out_dtype=torch.float32, outs=None, split: bool = True):
    """nf4_gemv_grouped_ws (split=True, with a workspace this call allocates)
    or nf4_gemv_grouped (split=False): several independent decode products in
    one call. xs[i] is [M, K_i] (same M and dtype for all), qss[i] the
    quantized [N_i, K_i] weight. Returns the list of y_i [M, N_i]."""
    count = len(xs)
    if count != len(qss) or count > GEMV_MAX_GROUP:
        raise ValueError("gemv_grouped takes matching lists of at most 16 problems")
    if count == 0:
        return []
    xs2, ys, descs, Ns, Ks = [], [], [], [], []
    for i, (x, qs) in enumerate(zip(xs, qss)):
        if x.dtype not in _DT or not x.is_cuda or len(qs.shape) != 2:
            raise TypeError("gemv_grouped expects GPU activations and [N, K] weights")
        N, K = (int(v) for v in qs.shape)
        x2 = _dev(x.reshape(-1, K))
        y = outs[i] if outs is not None else torch.empty((x2.shape[0], N), dtype=out_dtype,
                                                         device=x.device)
        xs2.append(x2)
        ys.append(y)
        descs.append(qs.desc())
        Ns.append(N)
        Ks.append(K)
    M = xs2[0].shape[0]
    Xarr = (ctypes.c_void_p * count)(*[t.data_ptr() for t in xs2])
    Yarr = (ctypes.c_void_p * count)(*[t.data_ptr() for t in ys])
    Darr = (QWeightDesc * count)(*descs)
    Narr = (ctypes.c_int32 * count)(*Ns)
    Karr = (ctypes.c_int32 * count)(*Ks)
    if not split:
        _check(lib().nf4_gemv_grouped(count, Xarr, M, Darr, Narr, Karr, _DT[xs2[0].dtype],
                                      _DT[ys[0].dtype], Yarr, _stream(xs2[0])),
               "nf4_gemv_grouped")
        return ys
    need = sum(workspace_bytes(M, qs, xs2[0].dtype, ys[0].dtype) for qs in qss)
    wp, wb, _keep = _workspace(need, xs2[0].device)
    _check(lib().nf4_gemv_grouped_ws(count, Xarr, M, Darr, Narr, Karr, _DT[xs2[0].dtype],
                                     _DT[ys[0].dtype], Yarr, wp, wb, _stream(xs2[0])),
           "nf4_gemv_grouped_ws")
    return ys


def gemm(x: torch.Tensor, qs: QuantState, out_dtype=torch.bfloat16, out=None) -> torch.Tensor:
    """nf4_gemm: y[M, N] = x[M, K] . cd(W)^T for any M (compute dtype = x's)."""
    return _product(lib().nf4_gemm, "nf4_gemm", x, qs, out_dtype, out)


def linear(x: torch.Tensor, qs: QuantState, bias: torch.Tensor | None = None,
           out_dtype=None, out=None, split: bool = True) -> torch.Tensor:
    """nf4_linear_ws (split=True, with a workspace this call allocates when
    nf4_linear_workspace_bytes asks for one) or nf4_linear_ex (split=False):
    y[M, N] = x[M, K] . cd(W)^T (+ bias[N] in the compute dtype, added in fp32
    before the output rounding); the compute dtype is x's dtype; M <= 64 runs
    the decode kernels, larger M the prefill GEMM. A 2-D x (or ``out``) with a
    row stride is passed in place. out_dtype defaults to the compute dtype."""
    if x.dtype not in _DT or not x.is_cuda:
        raise TypeError("nf4_linear expects bf16 / fp16 / fp32 activations on the GPU")
    if len(qs.shape) != 2:
        raise ValueError("nf4_linear expects a quantized [N, K] weight")
    N, K = (int(s) for s in qs.shape)
    if bias is not None:
        if bias.dtype != x.dtype or not bias.is_cuda or bias.numel() != N:
            raise ValueError("nf4_linear expects a GPU bias of N elements in x's dtype")
        bias = _dev(bias.reshape(-1))
    x2, ldx = _rows2d(x, K)
    M = x2.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or x.dtype, device=x.device)
    if out.dim() != 2 or out.shape != (M, N) or out.stride(1) != 1 or \
            (M > 1 and out.stride(0) < N) or out.data_ptr() % 16:
        raise ValueError("nf4_linear: out must be an [M, N] view with unit column stride")
    ldy = out.stride(0) if M > 1 else N
    d = qs.desc()
    if not split:
        _check(lib().nf4_linear_ex(_ptr(x2), ldx, M, ctypes.byref(d), N, K,
                                   None if bias is None else _ptr(bias), _DT[x.dtype],
                                   _DT[out.dtype], _ptr(out), ldy, _stream(x2)), "nf4_linear_ex")
        return out
    wp, wb, _keep = _workspace(workspace_bytes(M, qs, x.dtype, out.dtype), x.device)
    _check(lib().nf4_linear_ws(_ptr(x2), ldx, M, ctypes.byref(d), N, K,
                               None if bias is None else _ptr(bias), _DT[x.dtype], _DT[out.dtype],
                               _ptr(out), ldy, wp, wb, _stream(x2)), "nf4_linear_ws")
    return out


__all__ = [
    "QuantState", "QWeightDesc", "Nf4Error", "lib", "exported_names", "codebook", "packed_bytes",
    "num_blocks", "quantize", "quantize_grouped", "double_quant", "dequantize",
    "dequantize_grouped", "gemv", "gemv_grouped", "gemm", "linear", "workspace_bytes",
]
