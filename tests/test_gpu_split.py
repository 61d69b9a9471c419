"""GPU parity of the decode products for M up to 64 and of the K split.

Activations that do not fit the registers of one compute unit (8 <= M <= 16
with K > 6144, 17 <= M <= 32 with K > 4096, M > 32 with K > 2048) are split along K
when the caller brings a workspace (nf4_linear_ws, nf4_gemv_grouped_ws): each
K range is summed into fp32 partials and a second kernel adds the ranges in
order. Where that split would take two (M <= 16) or three (M > 16) or more
ranges, the tiled kernel (x staged in LDS, its own split) takes the product. Without a workspace the same products stream x (nf4_linear_ex). Both
are held to the product bar against the fp64 oracle: rel-L2 <= 1e-4 and
|y - y_ref| <= 1e-3 ||w_row|| ||x_row|| (+ 1e-3 |bias|), bf16 output = RNE of
the fp32-output run, repeated runs bitwise identical, and a grouped call equal
to the single calls bit for bit.
"""
import os

import numpy as np
import pytest
import torch

import workloads
from workloads import to_u16

pytestmark = pytest.mark.gpu

REL_L2 = 1e-4
PER_ELEM = 1e-3
THREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module")
def nf4():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_weight_quantization_nf4_amd as m

    assert m.lib().nf4_device_check() == 0, "device is not gfx950"
    return m


def dev(t):
    return t.to("cuda")


def u16_to_f64(a):
    return (np.asarray(a).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def quantized(nf4, orc, w, bs, qt, dq):
    """GPU quantization (checked bit-exact against the oracle) and the oracle's
    scale arrays for the products."""
    qs = nf4.quantize(dev(w), bs, qt, double_quant=dq)
    p_ref, a_ref = orc.quantize(to_u16(w.reshape(-1)), bs, qt)
    assert np.array_equal(qs.packed.cpu().numpy(), p_ref)
    sc = dict(absmax=a_ref)
    if dq:
        q_ref, s_ref = orc.double_quant(a_ref, 256)
        assert np.array_equal(qs.absmax_q.cpu().numpy(), q_ref)
        sc = dict(absmax_q=q_ref, absmax_scale=s_ref)
    return qs, p_ref, sc


def check(y32, y_ref, wrow_norm, x16, bias16=None):
    y = y32.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(y - y_ref) / max(np.linalg.norm(y_ref), 1e-300)
    assert rel <= REL_L2, f"relative L2 error {rel:.3e}"
    bound = PER_ELEM * np.outer(np.linalg.norm(u16_to_f64(x16), axis=1), wrow_norm)
    if bias16 is not None:
        bound = bound + PER_ELEM * np.abs(u16_to_f64(bias16))[None, :]
    err = np.abs(y - y_ref)
    assert np.all(err <= bound + 1e-30), f"max err/bound {np.max(err / (bound + 1e-30)):.3e}"
    return rel


def wc_norms(orc, packed, N, K, bs, qt, sc):
    _, wc16 = orc.dequantize(packed, N * K, bs, qt, **sc)
    return np.linalg.norm(u16_to_f64(wc16.reshape(N, K)), axis=1)


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
@pytest.mark.parametrize("which", [0, 1], ids=["up-11008x4096", "down-4096x11008"])
def test_linear_mlp_shapes_m17_to_64(nf4, orc, qt, which):
    """The MLP shapes (NF4 and FP4, bs 64 + double quant) at M = 17, 32, 48 and
    64 with a bias, every output against the oracle; with the workspace
    (split where the shape asks) and without (x streamed)."""
    m = workloads.MLP.matrices[which]
    w = m.make()
    N, K = w.shape
    qs, packed, sc = quantized(nf4, orc, w, 64, qt, True)
    x = workloads.MLP.activations(K, 64)
    x16 = to_u16(x)
    bias = workloads.normal_bf16((N,), 0.5, 31 + which)
    b16 = to_u16(bias)
    y_all = orc.gemv_quantized_threads(x16, packed, N, K, THREADS, 64, qt, **sc)
    y_all = y_all + u16_to_f64(b16)[None, :]
    wn = wc_norms(orc, packed, N, K, 64, qt, sc)
    for M in (17, 32, 48, 64):
        xd = dev(x[:M])
        for split in (True, False):
            y32 = nf4.linear(xd, qs, dev(bias), out_dtype=torch.float32, split=split)
            check(y32, y_all[:M], wn, x16[:M], b16)
            y16 = nf4.linear(xd, qs, dev(bias), out_dtype=torch.bfloat16, split=split)
            assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
            assert torch.equal(nf4.linear(xd, qs, dev(bias), out_dtype=torch.float32,
                                          split=split), y32), "not deterministic"


@pytest.mark.parametrize("bs", [32, 64, 128, 256])
@pytest.mark.parametrize("dq", [0, 1, 2])
def test_split_blocksizes_and_modes(nf4, orc, bs, dq):
    """K split with every block size (at 256 a K range can start inside a
    block), the three double-quant modes, ragged rows and a K that is not a
    multiple of the 128-code chunk; M across the three row-tile counts."""
    cases = [(37, 6144 + 2 * bs, 12), (50, 4096 + bs, 20), (29, 2048 + bs, 40), (64, 11008, 64)]
    for i, (N, K, M) in enumerate(cases):
        if K % bs:
            continue
        w = workloads.normal_bf16((N, K), 0.02, 6100 + 7 * i + bs)
        x = workloads.normal_bf16((M, K), 1.0, 6200 + 7 * i + bs)
        qs = nf4.quantize(dev(w), bs, "nf4", double_quant=dq)
        assert nf4.workspace_bytes(M, qs, torch.bfloat16, torch.float32) > 0, (N, K, M)
        p_ref, a_ref = orc.quantize(to_u16(w.reshape(-1)), bs, "nf4")
        sc = dict(absmax=a_ref)
        if dq == 1:
            q, s = orc.double_quant(a_ref, 256)
            sc = dict(absmax_q=q, absmax_scale=s)
        elif dq == 2:
            q, s, mu = orc.double_quant_centred(a_ref, 256)
            sc = dict(absmax_q=q, absmax_scale=s, absmax_offset=mu)
        x16 = to_u16(x)
        y_ref = orc.gemv_quantized_typed(x16, p_ref, N, K, bs, "nf4", **sc)
        _, wc16 = orc.dequantize(p_ref, N * K, bs, "nf4", **sc)
        wn = np.linalg.norm(u16_to_f64(wc16.reshape(N, K)), axis=1)
        y = nf4.gemv(dev(x), qs, torch.float32)
        check(y, y_ref, wn, x16)
        assert torch.equal(nf4.gemv(dev(x), qs, torch.float32), y)


def test_split_fp16_compute(nf4, orc):
    """fp16 activations and compute dtype on the split path (M = 12, K = 11008
    and M = 64, K = 4096)."""
    for (N, K, M) in [(300, 11008, 12), (200, 4096, 64)]:
        w = workloads.normal_bf16((N, K), 0.02, 7100 + K)
        qs, packed, sc = quantized(nf4, orc, w, 64, "nf4", True)
        x = torch.randn((M, K), generator=torch.Generator().manual_seed(7200 + M)).to(torch.float16)
        xh = x.view(torch.int16).numpy().view(np.uint16)
        y_ref = orc.gemv_quantized_typed(xh, packed, N, K, 64, "nf4", dtype="fp16", **sc)
        assert nf4.workspace_bytes(M, qs, torch.float16, torch.float32) > 0
        y = nf4.gemv(dev(x), qs, torch.float32)
        yy = y.cpu().numpy().astype(np.float64)
        assert np.linalg.norm(yy - y_ref) / np.linalg.norm(y_ref) <= REL_L2
        xn = np.linalg.norm(x.float().numpy().astype(np.float64), axis=1)
        _, wh = orc.dequantize(packed, N * K, 64, "nf4", half="fp16", **sc)
        wn = np.linalg.norm(orc.convert(wh, "fp16", "fp32").astype(np.float64).reshape(N, K),
                            axis=1)
        assert np.all(np.abs(yy - y_ref) <= PER_ELEM * np.outer(xn, wn))


def test_split_grouped_matches_single(nf4, orc):
    """A grouped call with a workspace over products of two K (two launches,
    one split) and two blocksizes at M = 16 and 64: each output equals the
    single call with a workspace bit for bit; a workspace one byte short of
    the query takes the streaming kernel, bitwise nf4_linear_ex."""
    shapes = [(4096, 4096, 64), (1000, 11008, 64), (257, 11008, 128), (300, 4096, 64)]
    for M in (16, 64):
        qss, xs = [], []
        for i, (N, K, bs) in enumerate(shapes):
            w = workloads.normal_bf16((N, K), 0.02, 7300 + i)
            qss.append(nf4.quantize(dev(w), bs, "nf4", double_quant=True))
            xs.append(dev(workloads.normal_bf16((M, K), 1.0, 7400 + i + M)))
        ys = nf4.gemv_grouped(xs, qss, torch.bfloat16)
        for y, x, qs in zip(ys, xs, qss):
            assert torch.equal(y.view(torch.int16), nf4.gemv(x, qs, torch.bfloat16).view(torch.int16))
    # an undersized workspace: the streaming kernel
    import ctypes

    N, K, M = 1000, 11008, 16
    w = workloads.normal_bf16((N, K), 0.02, 7500)
    qs = nf4.quantize(dev(w), 64, "nf4", double_quant=True)
    x = dev(workloads.normal_bf16((M, K), 1.0, 7501))
    need = nf4.workspace_bytes(M, qs, torch.bfloat16, torch.float32)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y_ex = nf4.linear(x, qs, out_dtype=torch.float32, split=False)
    y_small = torch.empty_like(y_ex)
    d = qs.desc()
    rc = nf4.lib().nf4_linear_ws(x.data_ptr(), K, M, ctypes.byref(d), N, K, None, 0, 1,
                                 y_small.data_ptr(), N, ws.data_ptr(), need - 1,
                                 torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    assert torch.equal(y_small, y_ex)
    y_full = torch.empty_like(y_ex)
    rc = nf4.lib().nf4_linear_ws(x.data_ptr(), K, M, ctypes.byref(d), N, K, None, 0, 1,
                                 y_full.data_ptr(), N, ws.data_ptr(), need,
                                 torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    assert torch.equal(y_full, nf4.linear(x, qs, out_dtype=torch.float32))


def test_gemv_7b_layer_m64_split(nf4, orc):
    """One 7B layer's seven products (4 x [4096, 4096], 3 x [11008, 4096]) in
    one grouped call at M = 64 (each split in two K ranges): sampled rows of
    every product against the oracle, each product bitwise its single call."""
    shapes = [(4096, 4096)] * 4 + [(11008, 4096)] * 3
    M = 64
    qss, xs, refs = [], [], []
    rng = np.random.default_rng(99)
    for j, (N, K) in enumerate(shapes):
        w = workloads.normal_bf16((N, K), 0.02, 5000 + j)
        qs, packed, sc = quantized(nf4, orc, w, 64, "nf4", True)
        x = workloads.normal_bf16((M, K), 1.0, 6000 + j)
        rows = np.sort(rng.choice(N, 96, replace=False))
        # the oracle on the sampled rows only: their codes and scales
        _, wc16 = orc.dequantize(packed, N * K, 64, "nf4", **sc)
        wc = wc16.reshape(N, K)[rows]
        refs.append((rows, orc.matmul_bf16(to_u16(x), wc),
                     np.linalg.norm(u16_to_f64(wc), axis=1), to_u16(x)))
        qss.append(qs)
        xs.append(dev(x))
    ys = nf4.gemv_grouped(xs, qss, torch.float32)
    for y, x, qs, (rows, y_ref, wn, x16) in zip(ys, xs, qss, refs):
        assert torch.equal(y, nf4.gemv(x, qs, torch.float32))
        check(y[:, torch.as_tensor(rows, device="cuda")], y_ref, wn, x16)


def test_tiled_decode_ragged_modes_and_groups(nf4, orc):
    """The tiled decode kernel (8..16 rows whose x would take two or more K
    ranges in registers, 64-row blocks; 17..64 rows with three or more, 128-row
    blocks): ragged N (a partial block), K that ends
    inside a 128-code chunk and ranges with an odd number of chunks, the three
    double-quant modes, bf16 and fp16 compute, every output against the
    oracle; the 16-bit output equals the rounding of the fp32 run, repeated
    runs are bitwise equal, and a grouped call over two products of one K
    equals the single calls bit for bit."""
    cases = [  # N, K, M, blocksize, double-quant mode, compute dtype
        (200, 8352, 17, 32, 2, "bf16"),   # 66 chunks, the last a quarter; 8 ranges of <= 9
        (131, 5184, 33, 64, 1, "fp16"),   # 41 chunks, the last a half; 2 blocks, the second of 3 rows
        (4097, 4224, 64, 128, 0, "bf16"), # 33 chunks; 33 blocks, the last of 1 row
        (70, 8384, 8, 64, 1, "bf16"),     # 8 rows, 66 chunks, the last a half; 2 blocks of 64, the second of 6 rows
        (131, 7232, 12, 32, 2, "fp16"),   # 57 chunks, the last a half; 3 blocks, the last of 3 rows
    ]
    for i, (N, K, M, bs, dq, ct) in enumerate(cases):
        ws = []
        for j, n in enumerate((N, N + 40)):
            w = workloads.normal_bf16((n, K), 0.02, 8100 + 10 * i + j)
            qs = nf4.quantize(dev(w), bs, "nf4", double_quant=dq)
            p_ref, a_ref = orc.quantize(to_u16(w.reshape(-1)), bs, "nf4")
            sc = dict(absmax=a_ref)
            if dq == 1:
                q, s = orc.double_quant(a_ref, 256)
                sc = dict(absmax_q=q, absmax_scale=s)
            elif dq == 2:
                q, s, mu = orc.double_quant_centred(a_ref, 256)
                sc = dict(absmax_q=q, absmax_scale=s, absmax_offset=mu)
            ws.append((qs, p_ref, sc, n))
        g = torch.Generator().manual_seed(8200 + i)
        if ct == "fp16":
            x = torch.randn((M, K), generator=g).to(torch.float16)
            xh = x.view(torch.int16).numpy().view(np.uint16)
            half, out16 = "fp16", torch.float16
        else:
            x = workloads.normal_bf16((M, K), 1.0, 8200 + i)
            xh = to_u16(x)
            half, out16 = "bf16", torch.bfloat16
        xn = np.linalg.norm(orc.convert(xh, half, "fp32").astype(np.float64).reshape(M, K), axis=1)
        xd = dev(x)
        singles = []
        for qs, p_ref, sc, n in ws:
            assert nf4.workspace_bytes(M, qs, x.dtype, torch.float32) > 0, (n, K, M)
            y_ref = orc.gemv_quantized_typed(xh, p_ref, n, K, bs, "nf4", dtype=half, **sc)
            _, wh = orc.dequantize(p_ref, n * K, bs, "nf4", half=half, **sc)
            wn = np.linalg.norm(orc.convert(wh, half, "fp32").astype(np.float64).reshape(n, K),
                                axis=1)
            y = nf4.gemv(xd, qs, torch.float32)
            yy = y.cpu().numpy().astype(np.float64)
            rel = np.linalg.norm(yy - y_ref) / np.linalg.norm(y_ref)
            assert rel <= REL_L2, (i, n, rel)
            assert np.all(np.abs(yy - y_ref) <= PER_ELEM * np.outer(xn, wn)), (i, n)
            assert torch.equal(nf4.gemv(xd, qs, torch.float32), y), "not deterministic"
            y16 = nf4.gemv(xd, qs, out16)
            assert torch.equal(y16.view(torch.int16), y.to(out16).view(torch.int16))
            singles.append(y16)
        ys = nf4.gemv_grouped([xd, xd], [ws[0][0], ws[1][0]], out16)
        for y, y1 in zip(ys, singles):
            assert torch.equal(y.view(torch.int16), y1.view(torch.int16))


def test_tiled_decode_strided_x_and_y(nf4, orc):
    """The tiled kernel's products on a row-strided activation slice, writing
    (through the summing kernel) into a row-strided output window with a
    bias: bitwise the contiguous call, the rest of the output buffer
    untouched, and within the bar of the oracle."""
    N, K, M = 300, 8256, 24  # 65 chunks: three K ranges of the register-resident split
    w = workloads.normal_bf16((N, K), 0.02, 8301)
    qs, packed, sc = quantized(nf4, orc, w, 64, "nf4", True)
    big = workloads.normal_bf16((M, K + 64), 1.0, 8302)
    x = dev(big)[:, 32:32 + K]
    bias = workloads.normal_bf16((N,), 0.5, 8303)
    for out_dtype in (torch.float32, torch.bfloat16):
        ref = nf4.linear(x.contiguous(), qs, dev(bias), out_dtype)
        out = torch.full((M, N + 24), 7.0, device="cuda", dtype=out_dtype)
        win = out[:, 8:8 + N]
        nf4.linear(x, qs, dev(bias), out_dtype, out=win)
        assert torch.equal(win, ref)
        assert torch.all(out[:, :8] == 7.0) and torch.all(out[:, 8 + N:] == 7.0)
    x16 = to_u16(big[:, 32:32 + K].contiguous())
    b16 = to_u16(bias)
    y_ref = orc.gemv_quantized_threads(x16, packed, N, K, THREADS, 64, "nf4", **sc)
    y_ref = y_ref + u16_to_f64(b16)[None, :]
    check(nf4.linear(x, qs, dev(bias), torch.float32), y_ref, wc_norms(orc, packed, N, K, 64, "nf4", sc),
          x16, b16)
