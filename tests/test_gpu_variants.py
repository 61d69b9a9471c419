"""GPU parity of the variants: decode batches up to M = 64, the fp16 and fp32
compute dtypes, fp16 dequantization, fp16 / fp32 / strided quantize inputs,
the mean-centred double quantization and strided activations / outputs --
each through the C ABI (thin binding) against the CPU oracle.

Bar (as for the bf16 path): codes, scales, double-quant bytes and
dequantized values bit-exact; products within relative L2 <= 1e-4 and, per
element, |y - y_ref| <= 1e-3 ||w_row|| ||x_row|| (+ 1e-3 |bias|) of the fp64
oracle in the same compute dtype; repeated calls bitwise identical.
"""
import numpy as np
import pytest
import torch

import workloads
from workloads import to_u16

pytestmark = pytest.mark.gpu

REL_L2 = 1e-4
PER_ELEM = 1e-3
TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


@pytest.fixture(scope="module")
def nf4():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_weight_quantization_nf4_amd as m

    assert m.lib().nf4_device_check() == 0, "device is not gfx950"
    return m


def bits(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a CPU/GPU tensor: uint16 bits for 16-bit floats, the
    values for fp32."""
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "fp16":
        return a.view(np.float16).astype(np.float64)
    return a.astype(np.float64)


def rand_act(shape, dtype, seed, scale=1.0):
    x = workloads.normal_bf16(shape, scale, seed).float()
    return x.to(TORCH_DT[dtype])


def oracle_quant(orc, w_host: np.ndarray, dtype, bs, qt, mode):
    p, a = orc.quantize_typed(w_host, dtype, bs, qt)
    ref = dict(packed=p, absmax=a)
    if mode == 1:
        q, s2 = orc.double_quant(a, 256)
        ref.update(absmax_q=q, absmax_scale=s2)
    elif mode == 2:
        q, s2, mu = orc.double_quant_centred(a, 256)
        ref.update(absmax_q=q, absmax_scale=s2, absmax_offset=mu)
    return ref


def scales(ref, mode):
    if mode == 0:
        return dict(absmax=ref["absmax"])
    kw = dict(absmax_q=ref["absmax_q"], absmax_scale=ref["absmax_scale"])
    if mode == 2:
        kw["absmax_offset"] = ref["absmax_offset"]
    return kw


def check_state(qs, ref, mode):
    assert np.array_equal(qs.packed.cpu().numpy(), ref["packed"]), "packed codes differ"
    assert np.array_equal(qs.absmax.cpu().numpy().view(np.uint32), ref["absmax"].view(np.uint32))
    if mode:
        assert np.array_equal(qs.absmax_q.cpu().numpy(), ref["absmax_q"]), "absmax_q differs"
        assert np.array_equal(qs.absmax_scale.cpu().numpy().view(np.uint32),
                              ref["absmax_scale"].view(np.uint32))
    if mode == 2:
        assert np.array_equal(qs.absmax_offset.cpu().numpy().view(np.uint32),
                              ref["absmax_offset"].view(np.uint32)), "absmax_offset differs"


def check_product(y, y_ref, wc, dtype, x_host, bias_host=None):
    yy = y.float().cpu().numpy().astype(np.float64) if y.dtype != torch.float32 else \
        y.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(yy - y_ref) / max(np.linalg.norm(y_ref), 1e-300)
    wn = np.linalg.norm(to_f64(wc, dtype), axis=1)
    xn = np.linalg.norm(to_f64(x_host, dtype), axis=1)
    bound = PER_ELEM * np.outer(xn, wn)
    if bias_host is not None:
        bound = bound + PER_ELEM * np.abs(to_f64(bias_host, dtype))[None, :]
    if y.dtype != torch.float32:  # the output rounding itself
        bound = bound + 2.0 ** -8 * np.abs(y_ref)
    else:
        assert rel <= REL_L2, f"relative L2 error {rel:.3e}"
    err = np.abs(yy - y_ref)
    assert np.all(err <= bound + 1e-30), f"max err/bound {np.max(err / (bound + 1e-30)):.3e}"


def weight_and_ref(nf4, orc, N, K, bs, qt, mode, seed, cd="bf16"):
    """Quantize a seeded bf16 weight on the GPU and in the oracle (bit-exact
    check), and return the oracle's compute-dtype weights [N, K]."""
    w = workloads.normal_bf16((N, K), 0.02, seed)
    qs = nf4.quantize(w.cuda(), bs, qt, double_quant=mode)
    ref = oracle_quant(orc, to_u16(w).reshape(-1), "bf16", bs, qt, mode)
    check_state(qs, ref, mode)
    if cd == "fp32":
        wc, _ = orc.dequantize(ref["packed"], N * K, bs, qt, **scales(ref, mode))
    else:
        _, wc = orc.dequantize(ref["packed"], N * K, bs, qt, half=cd, **scales(ref, mode))
    return qs, ref, wc.reshape(N, K)


# ------------------------------------------------------- decode up to M = 64


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
@pytest.mark.parametrize("which", [0, 1], ids=["up-11008x4096", "down-4096x11008"])
def test_decode_batches_17_to_64_mlp(nf4, orc, qt, which):
    """The MLP shapes at M = 17, 32, 33, 48, 64 with a bias (nf4_linear) and
    without (nf4_gemv), against the oracle; the bias result is one fp32 add of
    the bias to the plain result."""
    m = workloads.MLP.matrices[which]
    N, K = m.rows, m.cols
    qs, ref, wc = weight_and_ref(nf4, orc, N, K, 64, qt, 1, m.seed)
    x = workloads.MLP.activations(K, 64)
    x16 = to_u16(x)
    b = workloads.normal_bf16((N,), 0.5, 4000 + which)
    y_all = orc.matmul_bf16(x16, wc)
    bf = to_f64(to_u16(b), "bf16")
    for M in (17, 32, 33, 48, 64):
        xd = x[:M].cuda()
        y = nf4.gemv(xd, qs, torch.float32)
        check_product(y, y_all[:M], wc, "bf16", x16[:M])
        yb = nf4.linear(xd, qs, b.cuda(), torch.float32)
        check_product(yb, y_all[:M] + bf[None, :], wc, "bf16", x16[:M], to_u16(b))
        assert torch.equal(yb, y + b.cuda().float()[None, :])
        assert torch.equal(nf4.gemv(xd, qs, torch.float32), y), "not deterministic"
        y16 = nf4.gemv(xd, qs, torch.bfloat16)
        assert torch.equal(y16.view(torch.int16), y.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_decode_ragged_shapes_all_m(nf4, orc, mode):
    """Ragged rows and K (a last chunk of fewer than 128 codes, K below one
    chunk per wave), every M tile count, mixed grouped shapes."""
    for (N, K, bs) in [(33, 96, 32), (100, 4160, 64), (17, 64, 64), (260, 1152, 128)]:
        qs, ref, wc = weight_and_ref(nf4, orc, N, K, bs, "nf4", mode, N + K)
        x = workloads.normal_bf16((64, K), 1.0, N * K)
        x16 = to_u16(x)
        y_all = orc.matmul_bf16(x16, wc)
        for M in (1, 2, 15, 16, 17, 31, 33, 47, 63, 64):
            y = nf4.gemv(x[:M].cuda(), qs, torch.float32)
            check_product(y, y_all[:M], wc, "bf16", x16[:M])


@pytest.mark.parametrize("M", [4, 40])
def test_decode_grouped_equals_single(nf4, orc, M):
    """A grouped call mixing K (4096 and 1024) and blocksizes: each product is
    bitwise its single call (one launch per K, results independent of the
    item size the group gets)."""
    shapes = [(4096, 4096, 64), (11008, 4096, 64), (500, 1024, 128), (4096, 4096, 64)]
    qss, xs = [], []
    for i, (N, K, bs) in enumerate(shapes):
        w = workloads.normal_bf16((N, K), 0.02, 60 + i)
        qss.append(nf4.quantize(w.cuda(), bs, "nf4", double_quant=True))
        xs.append(workloads.normal_bf16((M, K), 1.0, 70 + i).cuda())
    ys = nf4.gemv_grouped(xs, qss, torch.float32)
    for x, qs, y in zip(xs, qss, ys):
        assert torch.equal(y, nf4.gemv(x, qs, torch.float32))


# ------------------------------------------------------ compute dtypes


@pytest.mark.parametrize("cd", ["fp16", "fp32"])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_compute_dtypes_products(nf4, orc, cd, mode):
    """The decode kernels (M = 1, 5, 40), the GEMM (M = 70, 300) and the
    linear layer with a bias in the fp16 / fp32 compute dtype, against the
    oracle in that dtype; fp16 / bf16 / fp32 outputs."""
    N, K, bs = 300, 1024, 64
    qs, ref, wc = weight_and_ref(nf4, orc, N, K, bs, "nf4", mode, 91, cd=cd)
    x = rand_act((300, K), cd, 92)
    xh = bits(x)
    y_all = orc.matmul_typed(xh, wc, cd)
    b = rand_act((N,), cd, 93, 0.5)
    bh = bits(b)
    bf = to_f64(bh, cd)
    for M in (1, 5, 40, 70, 300):
        xd = x[:M].cuda()
        y = nf4.linear(xd, qs, None, torch.float32)
        check_product(y, y_all[:M], wc, cd, xh[:M])
        yb = nf4.linear(xd, qs, b.cuda(), torch.float32)
        check_product(yb, y_all[:M] + bf[None, :], wc, cd, xh[:M], bh)
        assert torch.equal(yb, y + b.cuda().float()[None, :])
        for od in (torch.float16, torch.bfloat16):
            yo = nf4.linear(xd, qs, None, od)
            assert torch.equal(yo, y.to(od)), (M, od)
        assert torch.equal(nf4.linear(xd, qs, None, torch.float32), y), "not deterministic"


def test_fp16_gemm_prefill_shape_sampled(nf4, orc):
    """fp16 compute at the prefill shape 2048 x 4096 x 14336 (NF4 bs 64 +
    double quant): 2048 sampled outputs against the oracle."""
    m = workloads.PREFILL.matrices[0]
    N, K = m.rows, m.cols
    qs, ref, wc = weight_and_ref(nf4, orc, N, K, 64, "nf4", 1, m.seed, cd="fp16")
    x = rand_act((2048, K), "fp16", 2004)
    xh = bits(x)
    y = nf4.gemm(x.cuda(), qs, torch.float32)
    rng = np.random.default_rng(9)
    ms, ns = rng.integers(0, 2048, 2048), rng.integers(0, N, 2048)
    ref_y = np.array([float(np.dot(to_f64(xh[i], "fp16"), to_f64(wc[j], "fp16")))
                      for i, j in zip(ms, ns)])
    got = y.cpu().numpy().astype(np.float64)[ms, ns]
    bound = PER_ELEM * np.linalg.norm(to_f64(wc[ns], "fp16"), axis=1) * np.linalg.norm(
        to_f64(xh[ms], "fp16"), axis=1)
    assert np.all(np.abs(got - ref_y) <= bound)
    assert np.linalg.norm(got - ref_y) / np.linalg.norm(ref_y) <= REL_L2


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_dequantize_fp16_and_centred(nf4, orc, mode, qt):
    """fp16 dequantization bit-exact (numpy's fp16 rounding of the fp32
    value), in every double-quant mode, fp32 and bf16 outputs too."""
    n = 64 * 4096 + 77
    w = workloads.normal_bf16((n,), 0.02, 123)
    qs = nf4.quantize(w.cuda(), 64, qt, double_quant=mode)
    ref = oracle_quant(orc, to_u16(w), "bf16", 64, qt, mode)
    check_state(qs, ref, mode)
    w32, w16 = orc.dequantize(ref["packed"], n, 64, qt, **scales(ref, mode))
    _, wh = orc.dequantize(ref["packed"], n, 64, qt, half="fp16", **scales(ref, mode))
    assert np.array_equal(bits(nf4.dequantize(qs, torch.float32)).view(np.uint32), w32.view(np.uint32))
    assert np.array_equal(bits(nf4.dequantize(qs, torch.bfloat16)), w16)
    assert np.array_equal(bits(nf4.dequantize(qs, torch.float16)), wh)


# ------------------------------------------------------- quantize inputs


@pytest.mark.parametrize("dtype", ["fp16", "fp32"])
@pytest.mark.parametrize("bs", [32, 64, 256, 1024])
def test_quantize_fp16_fp32_inputs(nf4, orc, dtype, bs):
    """fp16 / fp32 weights (values off the bf16 grid, outliers, ragged
    lengths) quantize bit-exactly as the oracle does on the same values."""
    for n in (bs * 300 + 13, 8 * bs, 5):
        w = (torch.randn(n, generator=torch.Generator().manual_seed(n + bs)) * 0.02)
        w[:: 97] *= 20.0
        w = w.to(TORCH_DT[dtype])
        for mode in (0, 1, 2):
            qs = nf4.quantize(w.cuda(), bs, "nf4", double_quant=mode)
            check_state(qs, oracle_quant(orc, bits(w), dtype, bs, "nf4", mode), mode)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_quantize_strided_rows(nf4, orc, dtype):
    """A [rows, cols] view with a row stride (a slice of a wider matrix) is
    quantized in place, bitwise as its contiguous copy."""
    base = (torch.randn(300, 1000, generator=torch.Generator().manual_seed(5)) * 0.02)
    base = base.to(TORCH_DT[dtype]).cuda()
    for sl in (base[:, 8:520], base[10:299, 16:992], base[:, 0:64]):
        for bs, mode in ((64, 1), (128, 2), (32, 0)):
            a = nf4.quantize(sl, bs, "nf4", double_quant=mode)
            b = nf4.quantize(sl.contiguous(), bs, "nf4", double_quant=mode)
            for k in ("packed", "absmax", "absmax_q", "absmax_scale", "absmax_offset"):
                ta, tb = getattr(a, k), getattr(b, k)
                assert (ta is None) == (tb is None)
                if ta is not None:
                    assert torch.equal(ta.view(torch.uint8), tb.view(torch.uint8)), (sl.shape, k)
    w = base[:, 8:520]
    check_state(nf4.quantize(w, 64, "nf4", double_quant=2),
                oracle_quant(orc, bits(w.contiguous()).reshape(-1), dtype, 64, "nf4", 2), 2)


def test_centred_double_quant_standalone(nf4, orc):
    """nf4_double_quant_ex in the centred mode at every blocksize2: bit-exact,
    including an all-equal group and a ragged last group."""
    rng = np.random.default_rng(17)
    for bs2 in (64, 128, 256, 512, 1024, 2048, 4096):
        for nb in (1, 3, bs2, bs2 + 5, 3 * bs2 + 77):
            a = (np.abs(rng.standard_normal(nb)) * 0.05).astype(np.float32)
            if nb > 2 * bs2:
                a[bs2:2 * bs2] = np.float32(0.04)
            q, s2, mu = nf4.double_quant(torch.from_numpy(a).cuda(), bs2, mode=2)
            q_r, s_r, m_r = orc.double_quant_centred(a, bs2)
            assert np.array_equal(q.cpu().numpy(), q_r), (bs2, nb)
            assert np.array_equal(s2.cpu().numpy().view(np.uint32), s_r.view(np.uint32))
            assert np.array_equal(mu.cpu().numpy().view(np.uint32), m_r.view(np.uint32))


# ------------------------------------------------------- strided products


@pytest.mark.parametrize("M", [1, 6, 40, 100])
def test_linear_strided_x_and_y(nf4, orc, M):
    """nf4_linear_ex on a row-strided activation slice writing into a
    row-strided output window: bitwise the contiguous result, and the rest of
    the output buffer is untouched."""
    N, K = 200, 512
    w = workloads.normal_bf16((N, K), 0.02, 3)
    qs = nf4.quantize(w.cuda(), 64, "nf4", double_quant=True)
    big = workloads.normal_bf16((M, K + 64), 1.0, 4).cuda()
    x = big[:, 32:32 + K]
    b = workloads.normal_bf16((N,), 0.5, 5).cuda()
    ref = nf4.linear(x.contiguous(), qs, b, torch.float32)
    out = torch.full((M, N + 24), 7.0, device="cuda")
    win = out[:, 8:8 + N]
    nf4.linear(x, qs, b, torch.float32, out=win)
    assert torch.equal(win, ref)
    assert torch.all(out[:, :8] == 7.0) and torch.all(out[:, 8 + N:] == 7.0)
