"""The torch.library operators and the Linear4bit module.

CPU: the module's life before quantization (construction, load_state_dict
from an nn.Linear, staying dense on the CPU), operator registration and the
fake (meta) implementations used for tracing. GPU: quantization on .to(cuda)
bit-exact against the oracle, the forward pass against the oracle's linear
layer in each compute dtype, torch.compile through the operators, and
torch.library.opcheck.
"""
import numpy as np
import pytest
import torch
from torch import nn

import workloads
from workloads import to_u16

from bit_weight_quantization_nf4_amd.ops import Linear4bit  # registers the nf4:: operators


def test_module_before_quantization():
    lin = nn.Linear(128, 64)
    q = Linear4bit(128, 64, compute_dtype=torch.bfloat16)
    q.load_state_dict(lin.state_dict())
    assert torch.equal(q.weight, lin.weight) and torch.equal(q.bias, lin.bias)
    q = q.to("cpu")
    assert not q.quantized and q.weight is not None
    with pytest.raises(RuntimeError):
        q(torch.randn(2, 128))
    assert "quantized=False" in repr(q)


def test_operators_registered_with_fake_impls():
    for name in ("quantize", "dequantize", "linear"):
        assert hasattr(torch.ops.nf4, name)
    w = torch.empty(64, 128, device="meta", dtype=torch.bfloat16)
    packed, absmax, q, s2, mu = torch.ops.nf4.quantize(w, 64, "nf4", 2)
    assert packed.shape == (4096,) and packed.dtype == torch.uint8
    assert absmax.shape == (128,) and q.shape == (128,) and s2.shape == (1,) and mu.shape == (1,)
    _, _, q0, s0, m0 = torch.ops.nf4.quantize(w, 64, "nf4", 0)
    assert q0.numel() == s0.numel() == m0.numel() == 0
    x = torch.empty(3, 5, 128, device="meta", dtype=torch.float16)
    y = torch.ops.nf4.linear(x, packed, absmax, q, s2, mu, None, 64, 128, 64, "nf4", 2)
    assert y.shape == (3, 5, 64) and y.dtype == torch.float16
    d = torch.ops.nf4.dequantize(packed, absmax, q, s2, mu, [64, 128], 64, "nf4", 2, torch.float16)
    assert d.shape == (64, 128) and d.dtype == torch.float16


# --------------------------------------------------------------------- GPU


def _oracle_layer(orc, w_bits, dtype, bs, qt, mode, N, K, cd):
    p, a = orc.quantize_typed(w_bits, dtype, bs, qt)
    kw = dict(absmax=a)
    if mode == 1:
        q, s2 = orc.double_quant(a, 256)
        kw = dict(absmax_q=q, absmax_scale=s2)
    elif mode == 2:
        q, s2, mu = orc.double_quant_centred(a, 256)
        kw = dict(absmax_q=q, absmax_scale=s2, absmax_offset=mu)
    if cd == "fp32":
        wc, _ = orc.dequantize(p, N * K, bs, qt, **kw)
    else:
        _, wc = orc.dequantize(p, N * K, bs, qt, half=cd, **kw)
    return p, a, kw, wc.reshape(N, K)


def _host(t):
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _f64(a, dt):
    if dt == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dt == "fp16":
        return a.view(np.float16).astype(np.float64)
    return a.astype(np.float64)


@pytest.mark.gpu
@pytest.mark.parametrize("cd,wdt,mode", [("bf16", torch.bfloat16, 1), ("fp16", torch.float16, 1),
                                         ("fp16", torch.float16, 2), ("fp32", torch.float32, 0)])
def test_linear4bit_quantizes_on_to_cuda_and_matches_oracle(orc, cd, wdt, mode):
    """The pages' flow: dense fp16/bf16 weights loaded, then .to("cuda")
    quantizes; the stored codes and scales are the oracle's, and the forward
    pass (bias fused) is within the product tolerance of the oracle."""
    import bit_weight_quantization_nf4_amd  # noqa: F401

    dt = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[wdt]
    cdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[cd]
    N, K = 320, 512
    lin = nn.Linear(K, N).to(wdt)
    with torch.no_grad():
        lin.weight.copy_((workloads.normal_bf16((N, K), 0.02, 21).float()).to(wdt))
        lin.bias.copy_((workloads.normal_bf16((N,), 0.5, 22).float()).to(wdt))
    q = Linear4bit(K, N, compute_dtype=cdt, double_quant=mode, dtype=wdt)
    q.load_state_dict(lin.state_dict())
    q = q.to("cuda")
    assert q.quantized and q.weight is None
    p, a, kw, wc = _oracle_layer(orc, _host(lin.weight).reshape(-1), dt, 64, "nf4", mode, N, K, cd)
    assert np.array_equal(q.weight_packed.cpu().numpy(), p)
    assert np.array_equal(q.weight_absmax.cpu().numpy().view(np.uint32), a.view(np.uint32))
    b_host = _host(lin.bias.to(cdt))
    for M in (1, 7, 100):
        x = (workloads.normal_bf16((M, K), 1.0, 23 + M).float()).to(cdt)
        y = q(x.cuda())
        assert y.dtype == cdt and y.shape == (M, N)
        y32 = torch.ops.nf4.linear(x.cuda(), q.weight_packed, q.weight_absmax, q.weight_absmax_q,
                                   q.weight_absmax_scale, q.weight_absmax_offset, q.bias, N, K,
                                   64, "nf4", mode)
        assert torch.equal(y, y32)
        ref = orc.matmul_typed(_host(x), wc, cd) + _f64(b_host, cd)[None, :]
        got = y.float().cpu().numpy().astype(np.float64)
        bound = 1e-3 * np.outer(np.linalg.norm(_f64(_host(x), cd), axis=1),
                                np.linalg.norm(_f64(wc, cd), axis=1))
        bound += 1e-3 * np.abs(_f64(b_host, cd))[None, :] + (0 if cd == "fp32" else 2 ** -7 * np.abs(ref))
        assert np.all(np.abs(got - ref) <= bound)
    sd = q.state_dict()
    assert "weight" not in sd and "weight_packed" in sd and "bias" in sd


@pytest.mark.gpu
def test_torch_compile_through_the_operators():
    """A small model of Linear4bit layers under torch.compile gives bitwise the
    eager result (the operators are opaque to the compiler; their fake
    implementations carry the shapes)."""
    torch.manual_seed(0)
    model = nn.Sequential(Linear4bit(256, 512, compute_dtype=torch.bfloat16), nn.GELU(),
                          Linear4bit(512, 128, compute_dtype=torch.bfloat16)).to("cuda")
    x = torch.randn(4, 9, 256, device="cuda", dtype=torch.bfloat16)
    eager = model(x)
    compiled = torch.compile(model)
    assert torch.equal(compiled(x), eager)
    assert torch.equal(compiled(x), eager)


@pytest.mark.gpu
def test_opcheck():
    w = workloads.normal_bf16((64, 256), 0.02, 3).cuda()
    torch.library.opcheck(torch.ops.nf4.quantize.default, (w, 64, "nf4", 1),
                          test_utils=("test_schema", "test_faketensor"))
    packed, absmax, q, s2, mu = torch.ops.nf4.quantize(w, 64, "nf4", 1)
    x = workloads.normal_bf16((3, 256), 1.0, 4).cuda()
    torch.library.opcheck(torch.ops.nf4.linear.default,
                          (x, packed, absmax, q, s2, mu, None, 64, 256, 64, "nf4", 1),
                          test_utils=("test_schema", "test_faketensor"))
    torch.library.opcheck(torch.ops.nf4.dequantize.default,
                          (packed, absmax, q, s2, mu, [64, 256], 64, "nf4", 1, torch.bfloat16),
                          test_utils=("test_schema", "test_faketensor"))
