"""nf4_linear_noalloc (the linear layer for callers that cannot allocate: its
K-split workspace is a static per-device array) against nf4_linear_ws, the
entry point whose kernels take the workspace from the caller: bitwise equal
outputs on two calls in a row, the second smaller, through the C ABI, and
within the product bar of the fp64 oracle; a product needing more than the
static scratch is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from workloads import to_u16

pytestmark = pytest.mark.gpu

SCRATCH = 32 << 20
NF4_ERR_SCRATCH = 5


@pytest.fixture(scope="module")
def nf4():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_weight_quantization_nf4_amd as m

    assert m.lib().nf4_device_check() == 0, "device is not gfx950"
    return m


def _u16_f64(a):
    return (np.asarray(a).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _noalloc(nf4, x, qs, bias, out):
    M, K = x.shape
    N = out.shape[1]
    d = qs.desc()
    return nf4.lib().nf4_linear_noalloc(
        x.data_ptr(), K, M, ctypes.byref(d), N, K, None if bias is None else bias.data_ptr(),
        0, 1 if out.dtype == torch.float32 else 0, out.data_ptr(), N,
        torch.cuda.current_stream().cuda_stream)


def _ws(nf4, x, qs, bias, out):
    M, K = x.shape
    N = out.shape[1]
    need = nf4.workspace_bytes(M, qs, x.dtype, out.dtype)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    d = qs.desc()
    rc = nf4.lib().nf4_linear_ws(
        x.data_ptr(), K, M, ctypes.byref(d), N, K, None if bias is None else bias.data_ptr(),
        0, 1 if out.dtype == torch.float32 else 0, out.data_ptr(), N, ws.data_ptr(), need,
        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return rc, need


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_matches_workspace_entry_point(nf4, orc, out_dtype):
    # first call: M = 64 over [4096, 11008] (six K ranges, 6 MiB of partials);
    # second, smaller: M = 16 over [1000, 11008] (two K ranges); third: a
    # product that needs no workspace (M = 4, K = 4096); fourth: a prefill
    # product that nf4_linear_ws runs on a dequantized weight and the static
    # scratch variant through the fused GEMM (the same bits)
    cases = [(64, 4096, 11008, 11), (16, 1000, 11008, 12), (4, 512, 4096, 13),
             (1600, 1000, 1088, 14)]
    for M, N, K, seed in cases:
        w = workloads.normal_bf16((N, K), 0.02, 8800 + seed)
        x = workloads.normal_bf16((M, K), 1.0, 8900 + seed)
        b = workloads.normal_bf16((N,), 0.5, 9000 + seed)
        qs = nf4.quantize(w.cuda(), 64, "nf4", double_quant=True)
        xd, bd = x.cuda(), b.cuda()
        y_ws = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
        rc, need = _ws(nf4, xd, qs, bd, y_ws)
        assert rc == 0
        assert need <= SCRATCH
        y_na = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
        assert _noalloc(nf4, xd, qs, bd, y_na) == 0
        torch.cuda.synchronize()
        assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16)), (M, N, K)
        # the oracle bar on sampled rows (fp32 output only; bf16 = RNE of it)
        if out_dtype == torch.float32:
            p_ref, a_ref = orc.quantize(to_u16(w.reshape(-1)), 64, "nf4")
            q_ref, s_ref = orc.double_quant(a_ref, 256)
            _, wc16 = orc.dequantize(p_ref, N * K, 64, "nf4", absmax_q=q_ref, absmax_scale=s_ref)
            rows = np.arange(0, N, max(1, N // 64))
            wc = wc16.reshape(N, K)[rows]
            y_ref = orc.linear_bf16(to_u16(x), wc, to_u16(b)[rows])
            y = y_na.cpu().numpy().astype(np.float64)[:, rows]
            assert np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref) <= 1e-4
            bound = 1e-3 * (np.outer(np.linalg.norm(_u16_f64(to_u16(x)), axis=1),
                                     np.linalg.norm(_u16_f64(wc), axis=1))
                            + np.abs(_u16_f64(to_u16(b)[rows]))[None, :])
            assert np.all(np.abs(y - y_ref) <= bound)


def test_noalloc_refuses_more_than_the_scratch(nf4):
    # M = 64, K = 11008: six K ranges of 64 x N fp32 partials; N = 21846 needs
    # just over 32 MiB
    N, K, M = 21846, 11008, 64
    need = 6 * M * N * 4
    assert need > SCRATCH
    d = nf4.QWeightDesc(0x10000, 0x20000, 0x10000, 0x20000, N * K, 64, 0, 1, 256, None)
    assert nf4.lib().nf4_linear_workspace_bytes(M, N, K, 64, 0, 1, 1) == (need + 255) // 256 * 256
    rc = nf4.lib().nf4_linear_noalloc(0x10000, K, M, ctypes.byref(d), N, K, None, 0, 1, 0x20000, N,
                                      None)
    assert rc == NF4_ERR_SCRATCH
    assert b"NF4_ERR_SCRATCH" in nf4.lib().nf4_status_string(NF4_ERR_SCRATCH)
