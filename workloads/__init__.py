"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws numbers; it holds none of the quantization arithmetic.
Weights are N(0, sigma^2) draws rounded to bf16 (by torch's own fp32 -> bf16
conversion), standing in for the 7B-class checkpoints the pages name
(Llama-2-7b-chat-hf, LLaMA-7B), which are not available here. Activations are
N(0, 1) in bf16. All generation is on the CPU with torch.Generator, so the
oracle and the HIP path see the same bytes; bf16 data is returned as uint16
bit patterns (numpy) or as torch.bfloat16 tensors.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


def normal_bf16(shape, sigma: float, seed: int) -> torch.Tensor:
    """bf16 CPU tensor of N(0, sigma^2) draws from a seeded generator."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    n = int(np.prod(shape)) if len(shape) else 1
    x = torch.randn(n, generator=g, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(torch.bfloat16).reshape(shape)


def normal_bf16_with_outliers(shape, sigma: float, seed: int, frac: float, factor: float,
                              outlier_seed: int) -> torch.Tensor:
    """N(0, sigma^2) weights where round(frac * n) distinct entries, drawn with
    their own seed, are multiplied by `factor` before the bf16 rounding."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    n = int(np.prod(shape))
    x = torch.randn(n, generator=g, dtype=torch.float32).mul_(sigma)
    k = int(round(frac * n))
    go = torch.Generator(device="cpu").manual_seed(int(outlier_seed))
    idx = torch.randperm(n, generator=go)[:k]
    x[idx] *= factor
    return x.to(torch.bfloat16).reshape(shape)


def to_u16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (same memory layout)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def from_u16(a: np.ndarray) -> torch.Tensor:
    """numpy uint16 bit patterns -> bf16 CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


@dataclass(frozen=True)
class Matrix:
    name: str
    rows: int  # N (output features)
    cols: int  # K (input features); quantization blocks run along K
    seed: int
    sigma: float = 0.02
    outlier_frac: float = 0.0
    outlier_factor: float = 1.0
    outlier_seed: int = 0

    def make(self) -> torch.Tensor:
        if self.outlier_frac > 0:
            return normal_bf16_with_outliers((self.rows, self.cols), self.sigma, self.seed,
                                             self.outlier_frac, self.outlier_factor,
                                             self.outlier_seed)
        return normal_bf16((self.rows, self.cols), self.sigma, self.seed)


@dataclass(frozen=True)
class Config:
    name: str
    matrices: tuple
    blocksizes: tuple = (64,)
    double_quant: bool = True
    quant_types: tuple = ("nf4",)
    ms: tuple = (1,)
    x_seed: int = 2000
    notes: str = field(default="", compare=False)

    def activations(self, K: int, M: int, salt: int = 0) -> torch.Tensor:
        return normal_bf16((M, K), 1.0, self.x_seed + 17 * M + salt)


# The five workloads (sizes and seeds). Weight layout is [N, K] row-major, the
# nn.Linear (out, in) convention; "K x N" in a prefill shape names the
# contraction only.
TINY = Config(
    name="tiny-256x512",
    matrices=(Matrix("w", 256, 512, seed=1001),),
    blocksizes=(64,), double_quant=False, ms=(1,), x_seed=2001,
    notes="NF4 bs64, no double quant; quantize, dequantize, GEMV M=1")

SQUARE_OUTLIERS = Config(
    name="square-4096-outliers",
    matrices=(Matrix("w", 4096, 4096, seed=1002, outlier_frac=0.001, outlier_factor=20.0,
                     outlier_seed=3002),),
    blocksizes=(64,), double_quant=True, ms=(1,), x_seed=2002,
    notes="NF4 bs64 + double quant (256); 0.1% outliers x20; decode GEMV M=1")

MLP = Config(
    name="mlp-11008x4096",
    matrices=(Matrix("up", 11008, 4096, seed=1003), Matrix("down", 4096, 11008, seed=1013)),
    blocksizes=(64,), double_quant=True, quant_types=("nf4", "fp4"), ms=(1, 4, 8, 16),
    x_seed=2003,
    notes="NF4 and FP4, bs64 + double quant; batched decode GEMV M in {1,4,8,16}")

PREFILL = Config(
    name="prefill-2048x4096x14336",
    matrices=(Matrix("w", 14336, 4096, seed=1004),),
    blocksizes=(64,), double_quant=True, ms=(2048,), x_seed=2004,
    notes="NF4 bs64 + double quant; X[2048, 4096] bf16 times W[14336, 4096]; fp32 accumulate")


def stack_7b(layers: int = 32) -> Config:
    """7B-shaped stack: each layer has four [4096, 4096] and three [11008, 4096]
    weights, independent seeds per matrix."""
    mats = []
    for layer in range(layers):
        for j in range(7):
            rows = 4096 if j < 4 else 11008
            mats.append(Matrix(f"l{layer}.w{j}", rows, 4096, seed=5000 + 7 * layer + j))
    return Config(name="stack-7b", matrices=tuple(mats), blocksizes=(64, 128, 256),
                  double_quant=True, ms=(1,), x_seed=6000,
                  notes="32 layers x (4 x [4096,4096] + 3 x [11008,4096]); bs sweep 64/128/256")


STACK_7B = stack_7b()

CONFIGS = {c.name: c for c in (TINY, SQUARE_OUTLIERS, MLP, PREFILL, STACK_7B)}
