"""GPU parity of the prefill path that dequantizes the weight once.

With a workspace (nf4_linear_ws) a product of at least 1536 rows dequantizes
W once into it, to the compute dtype (the dequantize kernel's values), and
runs the GEMM on the dequantized weight; without one (nf4_linear_ex,
nf4_gemm) the GEMM dequantizes each weight tile itself. Both run the same
tiles and the same MFMA order on the same bf16 / fp16 weights, so the results
must be equal bit for bit; each is also held to the product bar against the
fp64 oracle (rel-L2 <= 1e-4, |y - y_ref| <= 1e-3 ||w_row|| ||x_row||
(+ 1e-3 |bias|)).
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from workloads import to_u16

pytestmark = pytest.mark.gpu

REL_L2 = 1e-4
PER_ELEM = 1e-3
MIN_M = 1536  # the smallest M that takes the dequantized-weight path


@pytest.fixture(scope="module")
def nf4():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_weight_quantization_nf4_amd as m

    assert m.lib().nf4_device_check() == 0, "device is not gfx950"
    return m


def u16_to_f64(a):
    return (np.asarray(a).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def oracle_wc(orc, w, bs, qt, dq):
    """The oracle's quantization of w (bf16 [N, K]) and its bf16 dequantized
    weight; dq: 0 none, 1 symmetric double quant."""
    N, K = w.shape
    p_ref, a_ref = orc.quantize(to_u16(w.reshape(-1)), bs, qt)
    sc = dict(absmax=a_ref)
    if dq:
        q_ref, s_ref = orc.double_quant(a_ref, 256)
        sc = dict(absmax_q=q_ref, absmax_scale=s_ref)
    _, wc16 = orc.dequantize(p_ref, N * K, bs, qt, **sc)
    return p_ref, wc16.reshape(N, K)


def check_rows(orc, y32, x16, wc16, rows, b=None):
    """y32 [M, N] (fp32, on the GPU) against the oracle on the given rows of x
    (b: the bf16 bias bits, or None)."""
    y_ref = orc.linear_bf16(x16[rows], wc16, b)
    y = y32.cpu().numpy().astype(np.float64)[rows]
    rel = np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref)
    assert rel <= REL_L2, f"relative L2 error {rel:.3e}"
    bound = PER_ELEM * np.outer(np.linalg.norm(u16_to_f64(x16[rows]), axis=1),
                                np.linalg.norm(u16_to_f64(wc16), axis=1))
    if b is not None:
        bound = bound + PER_ELEM * np.abs(u16_to_f64(b))[None, :]
    assert np.all(np.abs(y - y_ref) <= bound), \
        f"max err/bound {np.max(np.abs(y - y_ref) / bound):.3e}"


@pytest.mark.parametrize("case", [
    # M, N, K, bs, qt, dq, bias: ragged M and N (N tiles not a multiple of 8)
    (1600, 1000, 1088, 64, "fp4", False, True),
    # N tiles a multiple of 8 (whole weight panels per XCD), bs 128 + DQ
    (1536, 1792, 2048, 128, "nf4", True, False),
    # K not a multiple of the 64-deep tile step (bs 32)
    (2000, 448, 1056, 32, "nf4", True, True),
])
def test_dequantized_weight_path_matches_fused_and_oracle(nf4, orc, case):
    M, N, K, bs, qt, dq, with_bias = case
    seed = M + N + K
    w = workloads.normal_bf16((N, K), 0.02, seed)
    x = workloads.normal_bf16((M, K), 1.0, seed + 1)
    b = workloads.normal_bf16((N,), 0.5, seed + 2) if with_bias else None
    qs = nf4.quantize(w.cuda(), bs, qt, double_quant=dq)
    p_ref, wc16 = oracle_wc(orc, w, bs, qt, dq)
    assert np.array_equal(qs.packed.cpu().numpy(), p_ref)
    assert nf4.workspace_bytes(M, qs, torch.bfloat16, torch.float32) == \
        (2 * N * K + 255) // 256 * 256
    xd = x.cuda()
    bd = None if b is None else b.cuda()
    for out_dtype in (torch.float32, torch.bfloat16):
        y_ws = nf4.linear(xd, qs, bd, out_dtype=out_dtype)                 # dequantized weight
        y_ex = nf4.linear(xd, qs, bd, out_dtype=out_dtype, split=False)    # fused GEMM
        torch.cuda.synchronize()
        assert torch.equal(y_ws.view(torch.int16), y_ex.view(torch.int16)), out_dtype
        if out_dtype == torch.float32:
            y32 = y_ws
            if b is None:
                assert torch.equal(nf4.gemm(xd, qs, torch.float32), y_ws)
        else:
            assert torch.equal(y_ws.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    rows = np.unique(np.concatenate([np.arange(0, M, 97), [M - 1]]))
    check_rows(orc, y32, to_u16(x), wc16, rows, None if b is None else to_u16(b))


def test_dequantized_weight_path_fp16_and_strides(nf4, orc):
    """fp16 compute with fp16 output, and row-strided x and y: bitwise the
    fused GEMM on the same views."""
    M, N, K = 1700, 672, 1024
    w = workloads.normal_bf16((N, K), 0.02, 5101)
    qs = nf4.quantize(w.cuda(), 64, "nf4", double_quant=True)
    xw = torch.randn((M, K + 64), generator=torch.Generator().manual_seed(5102)).half().cuda()
    x = xw[:, :K]
    yw_a = torch.full((M, N + 32), float("nan"), dtype=torch.float16, device="cuda")
    yw_b = torch.full((M, N + 32), float("nan"), dtype=torch.float16, device="cuda")
    nf4.linear(x, qs, out=yw_a[:, :N])
    nf4.linear(x, qs, out=yw_b[:, :N], split=False)
    torch.cuda.synchronize()
    assert torch.equal(yw_a[:, :N].view(torch.int16), yw_b[:, :N].view(torch.int16))
    assert torch.isnan(yw_a[:, N:]).all(), "wrote past the output view"
    # the fp16 result against the oracle (fp32 output, sampled rows)
    y32 = nf4.linear(x, qs, out_dtype=torch.float32)
    p_ref, a_ref = orc.quantize(to_u16(w.reshape(-1)), 64, "nf4")
    q_ref, s_ref = orc.double_quant(a_ref, 256)
    rows = np.arange(0, M, 113)
    xs = x.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)[rows]
    _, wc = orc.dequantize(p_ref, N * K, 64, "nf4", absmax_q=q_ref, absmax_scale=s_ref,
                           half="fp16")
    wc = wc.reshape(N, K)
    y_ref = orc.matmul_typed(xs, wc, "fp16")
    y = y32.cpu().numpy().astype(np.float64)[rows]
    assert np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref) <= REL_L2


def test_undersized_workspace_takes_the_fused_gemm(nf4):
    """A workspace below the query's size: the fused GEMM (nf4_linear_ex's
    bits); the query's size: the dequantized-weight path (the same bits)."""
    M, N, K = MIN_M, 448, 512
    w = workloads.normal_bf16((N, K), 0.02, 5201)
    qs = nf4.quantize(w.cuda(), 64, "nf4", double_quant=True)
    x = workloads.normal_bf16((M, K), 1.0, 5202).cuda()
    need = nf4.workspace_bytes(M, qs, torch.bfloat16, torch.float32)
    assert need == 2 * N * K
    assert nf4.workspace_bytes(M - 1, qs, torch.bfloat16, torch.float32) == 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y_ex = nf4.linear(x, qs, out_dtype=torch.float32, split=False)
    d = qs.desc()
    stream = torch.cuda.current_stream().cuda_stream
    for nbytes in (need - 256, need):
        y = torch.full_like(y_ex, float("nan"))
        rc = nf4.lib().nf4_linear_ws(x.data_ptr(), K, M, ctypes.byref(d), N, K, None, 0, 1,
                                     y.data_ptr(), N, ws.data_ptr(), nbytes, stream)
        assert rc == 0
        torch.cuda.synchronize()
        assert torch.equal(y, y_ex), nbytes
