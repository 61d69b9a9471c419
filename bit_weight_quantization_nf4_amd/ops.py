"""torch.library operators over the C ABI, and a ``Linear4bit``-style module.

[gitcode page on the bitsandbytes 0.46.0 release, section on the custom-op
 rework: the quantized operations are functional operators registered with
 ``torch.library`` so that ``torch.compile`` can trace through them; usage
 page icman.com.cn/news/48546, "Core Usage 3": ``Linear4bit(in, out,
 quant_type, compute_dtype)`` takes fp16/bf16 weights and quantizes them when
 the module is moved to the device; "Configuration": the compute dtype is the
 dtype the 4-bit weights are dequantized to.]

Operators (namespace ``nf4``), each a thin wrapper of one binding call -- no
arithmetic of the method runs in Python:
  nf4::quantize(Tensor w, int blocksize, str quant_type, int double_quant)
      -> (packed, absmax, absmax_q, absmax_scale, absmax_offset)
  nf4::dequantize(packed, absmax, absmax_q, absmax_scale, absmax_offset,
      int[] shape, int blocksize, str quant_type, int double_quant,
      ScalarType dtype) -> Tensor
  nf4::linear(Tensor x, packed, absmax, absmax_q, absmax_scale, absmax_offset,
      Tensor? bias, int N, int K, int blocksize, str quant_type,
      int double_quant) -> Tensor
Scale tensors a double-quant mode does not use are passed as empty tensors.
Each operator has a fake (meta) implementation for tracing. The operators
are inference operators: no autograd formula is registered.
"""
from __future__ import annotations

import math

import torch
from torch import nn

from . import QuantState, _dq, dequantize as _dequantize, linear as _linear, \
    quantize as _quantize


def _state(packed, absmax, absmax_q, absmax_scale, absmax_offset, shape, blocksize, quant_type,
           double_quant) -> QuantState:
    mode = _dq(double_quant)
    return QuantState(packed, absmax, absmax_q if mode else None,
                      absmax_scale if mode else None, tuple(int(s) for s in shape), int(blocksize),
                      quant_type, mode, 256, absmax_offset if mode == 2 else None)


def _sizes(n: int, blocksize: int, mode: int):
    nb = (n + blocksize - 1) // blocksize
    ng = (nb + 255) // 256
    return nb, ng, (nb if mode else 0), (ng if mode else 0), (ng if mode == 2 else 0)


@torch.library.custom_op("nf4::quantize", mutates_args=())
def quantize_op(w: torch.Tensor, blocksize: int, quant_type: str,
                double_quant: int) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor,
                                            torch.Tensor, torch.Tensor]:
    qs = _quantize(w, blocksize, quant_type, double_quant)

    def or_empty(t, dtype):  # a distinct empty tensor each (outputs may not alias)
        return t if t is not None else torch.empty(0, dtype=dtype, device=w.device)

    return (qs.packed, qs.absmax, or_empty(qs.absmax_q, torch.int8),
            or_empty(qs.absmax_scale, torch.float32), or_empty(qs.absmax_offset, torch.float32))


@quantize_op.register_fake
def _(w, blocksize, quant_type, double_quant):
    n = w.numel()
    nb, ng, nq, ns, no = _sizes(n, blocksize, _dq(double_quant))
    e = w.new_empty
    return (e((n + 1) // 2, dtype=torch.uint8), e(nb, dtype=torch.float32),
            e(nq, dtype=torch.int8), e(ns, dtype=torch.float32), e(no, dtype=torch.float32))


@torch.library.custom_op("nf4::dequantize", mutates_args=())
def dequantize_op(packed: torch.Tensor, absmax: torch.Tensor, absmax_q: torch.Tensor,
                  absmax_scale: torch.Tensor, absmax_offset: torch.Tensor, shape: list[int],
                  blocksize: int, quant_type: str, double_quant: int,
                  dtype: torch.dtype) -> torch.Tensor:
    qs = _state(packed, absmax, absmax_q, absmax_scale, absmax_offset, shape, blocksize,
                quant_type, double_quant)
    return _dequantize(qs, dtype)


@dequantize_op.register_fake
def _(packed, absmax, absmax_q, absmax_scale, absmax_offset, shape, blocksize, quant_type,
      double_quant, dtype):
    return packed.new_empty(tuple(shape), dtype=dtype)


@torch.library.custom_op("nf4::linear", mutates_args=())
def linear_op(x: torch.Tensor, packed: torch.Tensor, absmax: torch.Tensor,
              absmax_q: torch.Tensor, absmax_scale: torch.Tensor, absmax_offset: torch.Tensor,
              bias: torch.Tensor | None, N: int, K: int, blocksize: int, quant_type: str,
              double_quant: int) -> torch.Tensor:
    qs = _state(packed, absmax, absmax_q, absmax_scale, absmax_offset, (N, K), blocksize,
                quant_type, double_quant)
    y = _linear(x.reshape(-1, K), qs, bias, out_dtype=x.dtype)
    return y.reshape(*x.shape[:-1], N)


@linear_op.register_fake
def _(x, packed, absmax, absmax_q, absmax_scale, absmax_offset, bias, N, K, blocksize,
      quant_type, double_quant):
    return x.new_empty((*x.shape[:-1], N))


class Linear4bit(nn.Module):
    """A linear layer whose weight is stored as NF4/FP4 4-bit codes with block
    scales (optionally double-quantized) once the module is on the GPU.

    Until then it holds a dense ``weight`` [out_features, in_features] (and
    ``bias``), so ``load_state_dict`` from an ``nn.Linear`` works; moving the
    module to a GPU (``.to("cuda")`` / ``.cuda()``) quantizes the weight there
    and replaces it by the buffers ``weight_packed``, ``weight_absmax``,
    ``weight_absmax_q``, ``weight_absmax_scale`` and ``weight_absmax_offset``.
    The forward pass casts its input to ``compute_dtype`` and runs nf4::linear
    (the bias, cast to the compute dtype, fused in); the output is in the
    compute dtype.
    """

    def __init__(self, in_features: int, out_features: int, bias: bool = True,
                 compute_dtype=torch.bfloat16, quant_type: str = "nf4", blocksize: int = 64,
                 double_quant=True, device=None, dtype=None):
        super().__init__()
        if compute_dtype not in (torch.bfloat16, torch.float16, torch.float32):
            raise ValueError("compute_dtype must be bf16, fp16 or fp32")
        self.in_features = in_features
        self.out_features = out_features
        self.compute_dtype = compute_dtype
        self.quant_type = quant_type
        self.blocksize = blocksize
        self.double_quant = _dq(double_quant)
        self.weight = nn.Parameter(torch.empty(out_features, in_features, device=device,
                                               dtype=dtype), requires_grad=False)
        if bias:
            self.bias = nn.Parameter(torch.empty(out_features, device=device, dtype=dtype),
                                     requires_grad=False)
        else:
            self.register_parameter("bias", None)
        # nn.Linear's default initialisation, for modules not loaded from a checkpoint
        nn.init.kaiming_uniform_(self.weight, a=math.sqrt(5))
        if self.bias is not None:
            bound = 1 / math.sqrt(in_features) if in_features > 0 else 0
            nn.init.uniform_(self.bias, -bound, bound)
        self.quantized = False
        if self.weight.is_cuda:
            self._quantize()

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}, quant_type={self.quant_type}, "
                f"compute_dtype={self.compute_dtype}, blocksize={self.blocksize}, "
                f"double_quant={self.double_quant}, quantized={self.quantized}")

    @torch.no_grad()
    def _quantize(self) -> None:
        w = self.weight.detach()
        if w.dtype not in (torch.bfloat16, torch.float16, torch.float32):
            w = w.float()
        packed, absmax, q, s2, mu = torch.ops.nf4.quantize(w.contiguous(), self.blocksize,
                                                           self.quant_type, self.double_quant)
        del self.weight
        self.register_parameter("weight", None)
        self.register_buffer("weight_packed", packed)
        self.register_buffer("weight_absmax", absmax)
        self.register_buffer("weight_absmax_q", q)
        self.register_buffer("weight_absmax_scale", s2)
        self.register_buffer("weight_absmax_offset", mu)
        if self.bias is not None:
            self.bias = nn.Parameter(self.bias.detach().to(self.compute_dtype), requires_grad=False)
        self.quantized = True

    def _apply(self, fn, recurse=True):
        super()._apply(fn, recurse)
        # quantization happens when the dense weight reaches the GPU
        if not self.quantized and self.weight is not None and self.weight.is_cuda:
            self._quantize()
        return self

    def quant_state(self) -> QuantState:
        if not self.quantized:
            raise RuntimeError("Linear4bit is quantized when moved to the GPU")
        return _state(self.weight_packed, self.weight_absmax, self.weight_absmax_q,
                      self.weight_absmax_scale, self.weight_absmax_offset,
                      (self.out_features, self.in_features), self.blocksize, self.quant_type,
                      self.double_quant)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if not self.quantized:
            raise RuntimeError("Linear4bit runs on the GPU: move it there with .to('cuda')")
        x = x.to(self.compute_dtype)
        bias = self.bias if self.bias is None else self.bias.to(self.compute_dtype)
        return torch.ops.nf4.linear(x, self.weight_packed, self.weight_absmax,
                                    self.weight_absmax_q, self.weight_absmax_scale,
                                    self.weight_absmax_offset, bias, self.out_features,
                                    self.in_features, self.blocksize, self.quant_type,
                                    self.double_quant)


__all__ = ["Linear4bit", "quantize_op", "dequantize_op", "linear_op"]
