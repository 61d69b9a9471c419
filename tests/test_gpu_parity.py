"""GPU parity: the HIP path (through the C ABI via the thin binding) against the
CPU oracle on the same seeded inputs.

Bar: packed codes, absmax, double-quant bytes and dequantized fp32/bf16 values
bit-exact; products in fp32 within relative L2 <= 1e-4 and, per element,
|y - y_ref| <= 1e-3 * ||W_c[n, :]|| * ||x[m, :]|| against the fp64 oracle; the
bf16-output run equal to RNE of the fp32-output run; repeated runs bitwise
identical.
"""
import numpy as np
import pytest
import torch

import workloads
from workloads import to_u16

pytestmark = pytest.mark.gpu

REL_L2 = 1e-4
PER_ELEM = 1e-3


@pytest.fixture(scope="module")
def nf4():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_weight_quantization_nf4_amd as m

    assert m.lib().nf4_device_check() == 0, "device is not gfx950"
    return m


def dev(t):
    return t.to("cuda")


def u16_to_f64(a):
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_quant(nf4, orc, w_cpu, bs, qt, dq):
    """Quantize on GPU and oracle; assert bit-exact outputs. Returns both."""
    qs = nf4.quantize(dev(w_cpu), bs, qt, double_quant=dq)
    w16 = to_u16(w_cpu.reshape(-1))
    p_ref, a_ref = orc.quantize(w16, bs, qt)
    p = qs.packed.cpu().numpy()
    a = qs.absmax.cpu().numpy()
    assert np.array_equal(p, p_ref), f"packed codes differ ({np.sum(p != p_ref)} bytes)"
    assert np.array_equal(a.view(np.uint32), a_ref.view(np.uint32)), "absmax differs"
    ref = dict(packed=p_ref, absmax=a_ref)
    if dq:
        q_ref, s_ref = orc.double_quant(a_ref, 256)
        assert np.array_equal(qs.absmax_q.cpu().numpy(), q_ref), "absmax_q differs"
        assert np.array_equal(qs.absmax_scale.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
        ref.update(absmax_q=q_ref, absmax_scale=s_ref)
    return qs, ref


def oracle_scales(ref, dq):
    if dq:
        return dict(absmax_q=ref["absmax_q"], absmax_scale=ref["absmax_scale"])
    return dict(absmax=ref["absmax"])


def check_dequant(nf4, orc, qs, ref, bs, qt, dq):
    n = qs.n
    w32_ref, w16_ref = orc.dequantize(ref["packed"], n, bs, qt, **oracle_scales(ref, dq))
    w32 = nf4.dequantize(qs, torch.float32).reshape(-1).cpu().numpy()
    w16 = to_u16(nf4.dequantize(qs, torch.bfloat16).reshape(-1).cpu())
    assert np.array_equal(w32.view(np.uint32), w32_ref.view(np.uint32)), "fp32 dequant differs"
    assert np.array_equal(w16, w16_ref), "bf16 dequant differs"
    return w16_ref


def check_product(y32, y16, ref, wc16, x16, bias16=None):
    """Tolerance bar against the fp64 oracle plus bf16 == RNE(fp32). With a
    bias, the per-element bound grows by |bias[j]| (the fp32 sum is rounded
    once more after the bias is added)."""
    y = y32.cpu().numpy().astype(np.float64)
    err = np.abs(y - ref)
    rel = np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300)
    assert rel <= REL_L2, f"relative L2 error {rel:.3e}"
    wn = np.linalg.norm(u16_to_f64(wc16), axis=1)
    xn = np.linalg.norm(u16_to_f64(x16), axis=1)
    bound = PER_ELEM * np.outer(xn, wn)
    if bias16 is not None:
        bound = bound + PER_ELEM * np.abs(u16_to_f64(bias16))[None, :]
    assert np.all(err <= bound + 1e-30), f"max err/bound {np.max(err / (bound + 1e-30)):.3e}"
    if y16 is not None:
        assert torch.equal(y16.cpu().view(torch.int16), y32.to(torch.bfloat16).cpu().view(torch.int16))
    return rel


# ----------------------------------------------------------------- quantize


@pytest.mark.parametrize("cfg", [workloads.TINY, workloads.SQUARE_OUTLIERS], ids=lambda c: c.name)
def test_quantize_dequant_small_configs(nf4, orc, cfg):
    m = cfg.matrices[0]
    w = m.make()
    for bs in cfg.blocksizes:
        qs, ref = check_quant(nf4, orc, w, bs, "nf4", cfg.double_quant)
        check_dequant(nf4, orc, qs, ref, bs, "nf4", cfg.double_quant)


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_quantize_dequant_mlp_config(nf4, orc, qt):
    for m in workloads.MLP.matrices:
        w = m.make()
        qs, ref = check_quant(nf4, orc, w, 64, qt, True)
        check_dequant(nf4, orc, qs, ref, 64, qt, True)


def _all_bf16_classes():
    a_bits = (0x3F80 | np.arange(128)).astype(np.uint16)
    allx = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    xf = (allx.astype(np.uint32) << 16).view(np.float32)
    blocks = []
    for ab in a_bits:
        af = (np.array([ab], np.uint32) << 16).view(np.float32)[0]
        xs = allx[np.isfinite(xf) & (np.abs(xf) <= af)]
        xs = np.concatenate([xs, np.zeros((-len(xs)) % 63, np.uint16)]).reshape(-1, 63)
        blocks.append(np.concatenate([np.full((xs.shape[0], 1), ab, np.uint16), xs], axis=1))
    return np.concatenate(blocks).reshape(-1)


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_quantize_every_bf16_class(nf4, orc, qt):
    """Every normal (x, a) significand/exponent class: the kernel's reciprocal
    normalisation and cell lookup give the oracle's codes everywhere."""
    w = workloads.from_u16(_all_bf16_classes())
    check_quant(nf4, orc, w, 64, qt, False)


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_quantize_extreme_scales(nf4, orc, qt):
    """Blocks whose absmax sits at or beyond the fast-path range, including
    bf16 subnormals and the largest finite values, plus all-zero blocks."""
    base = workloads.normal_bf16((40, 64), 1.0, 77).float().clamp(-3.5, 3.5)
    scales = [2.0 ** e for e in (-140, -133, -126, -110, -101, -100, -99, -60, 0, 60, 100,
                                 119, 120, 121, 125)]
    rows = [to_u16((base[i % 40] * s).to(torch.bfloat16)) for i, s in enumerate(scales)]
    rows.append(np.zeros(64, np.uint16))
    rows.append(np.full(64, 0x7F7F, np.uint16))  # largest finite bf16
    rows.append(np.concatenate([np.full(32, 0xFF7F, np.uint16), np.full(32, 0x7E96, np.uint16)]))
    rows.append(np.arange(1, 65, dtype=np.uint16))  # bf16 subnormals only
    w = workloads.from_u16(np.stack(rows))
    assert torch.isfinite(w.float()).all()
    check_quant(nf4, orc, w, 64, qt, True)


@pytest.mark.parametrize("bs", [32, 64, 128, 256, 512, 1024, 2048, 4096])
def test_quantize_blocksizes_and_ragged_lengths(nf4, orc, bs):
    for n in (3 * bs + 517, 2 * bs, bs - 8, 1, 2, 7, 9, 17, 63, 65, 513):
        if n <= 0:
            continue
        w = workloads.normal_bf16((n,), 0.02, 1000 + n)
        for qt in ("nf4", "fp4"):
            qs, ref = check_quant(nf4, orc, w, bs, qt, n > 300)
            check_dequant(nf4, orc, qs, ref, bs, qt, n > 300)


@pytest.mark.parametrize("bs", [64, 128, 256])
def test_quantize_with_double_quant_groups(nf4, orc, bs):
    """Quantization with double quantization in one pass: whole and ragged
    groups of 256 blocks, an all-zero group and one whose largest scale sits
    in its last block, and more groups than one launch has workgroups (each
    then loops over several groups). The 33.6M-element case also dequantizes,
    so the dequantize kernel's waves each take more than one tile."""
    g = 256 * bs
    for n in (g, 3 * g + 5 * bs + 17, 2 * g - 1, 2049 * g + 3 * bs + 1):
        w = workloads.normal_bf16((n,), 0.02, 31 * n + bs).float()
        w[g:2 * g] = 0.0
        if n > 3 * g:
            w[3 * g - 1] = 4.0
        qs, ref = check_quant(nf4, orc, w.to(torch.bfloat16), bs, "nf4", True)
        if n > 3 * g and bs == 64:
            check_dequant(nf4, orc, qs, ref, bs, "nf4", True)


@pytest.mark.parametrize("bs,dq,qt", [(64, True, "nf4"), (128, True, "fp4"), (256, True, "nf4"),
                                      (64, False, "nf4"), (32, True, "nf4"), (1024, True, "fp4")])
def test_quantize_grouped_matches_single(nf4, bs, dq, qt):
    """nf4_quantize_grouped writes, for every tensor, exactly what nf4_quantize
    writes for it alone: layer-sized tensors, a ragged tensor, an empty one,
    a single element."""
    sizes = [4096 * 4096, 0, 1000 * 512 + 37, 1, 11008 * 4096, 33 * 160]
    ws = [workloads.normal_bf16((n,), 0.02, 900 + i) for i, n in enumerate(sizes)]
    gpu = [dev(w) for w in ws]
    grouped = nf4.quantize_grouped(gpu, bs, qt, dq)
    for w, g in zip(gpu, grouped):
        single = nf4.quantize(w, bs, qt, double_quant=dq)
        keys = ("packed", "absmax", "absmax_q", "absmax_scale") if dq else ("packed", "absmax")
        for k in keys:
            a, b = getattr(g, k), getattr(single, k)
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (w.numel(), k)


def test_quantize_grouped_more_groups_than_workgroups(nf4):
    """A fused grouped launch whose groups of 256 blocks outnumber the
    launch's workgroup cap (16384): workgroups then walk several groups, of
    several tensors. Every tensor's output is bitwise its single-call one."""
    g = torch.Generator(device="cuda").manual_seed(5)
    n = 4096 * 4096 + 64 * 256  # 1025 groups at blocksize 64
    ws = [(torch.randn(n, device="cuda", generator=g) * 0.02).to(torch.bfloat16) for _ in range(16)]
    grouped = nf4.quantize_grouped(ws, 64, "nf4", True)
    for w, q in zip(ws, grouped):
        single = nf4.quantize(w, 64, "nf4", double_quant=True)
        for k in ("packed", "absmax", "absmax_q", "absmax_scale"):
            assert torch.equal(getattr(q, k).view(torch.uint8), getattr(single, k).view(torch.uint8)), k


@pytest.mark.parametrize("dq", [False, True])
def test_dequantize_grouped_matches_single(nf4, orc, dq):
    """nf4_dequantize_grouped: every output bitwise equal to nf4_dequantize of
    the tensor alone, for tensors of mixed blocksizes and sizes (whole tiles,
    a ragged tail, an empty tensor, tails only), fp32 and bf16 outputs; one
    small tensor is also checked against the oracle."""
    specs = [(4096 * 4096, 64), (0, 64), (1000 * 512 + 37, 128), (77, 32), (11008 * 4096, 64),
             (2048 + 513, 256)]
    qss = [nf4.quantize(dev(workloads.normal_bf16((n,), 0.02, 950 + i)), bs, "nf4",
                        double_quant=dq) for i, (n, bs) in enumerate(specs)]
    for dtype in (torch.bfloat16, torch.float32):
        ys = nf4.dequantize_grouped(qss, dtype)
        for qs, y in zip(qss, ys):
            assert torch.equal(y, nf4.dequantize(qs, dtype)), (qs.shape, dtype)
    w = workloads.normal_bf16((1000 * 512 + 37,), 0.02, 952)
    qs, ref = check_quant(nf4, orc, w, 128, "nf4", dq)
    _, w16_ref = orc.dequantize(ref["packed"], qs.n, 128, "nf4", **oracle_scales(ref, dq))
    y = nf4.dequantize_grouped([qss[0], qs], torch.bfloat16)[1]
    assert np.array_equal(to_u16(y.reshape(-1).cpu()), w16_ref)


def test_quantize_empty(nf4):
    qs = nf4.quantize(torch.empty(0, dtype=torch.bfloat16, device="cuda"), 64, "nf4", True)
    assert qs.packed.numel() == 0 and qs.absmax.numel() == 0


# ------------------------------------------------------------- double quant


@pytest.mark.parametrize("bs2", [64, 128, 256, 512, 1024, 2048, 4096])
def test_double_quant(nf4, orc, bs2):
    rng = np.random.default_rng(bs2)
    for nb in (1, 3, bs2 - 1, bs2, bs2 + 1, 5 * bs2 + 37):
        a = (np.abs(rng.standard_normal(nb)) * 0.05).astype(np.float32)
        if nb > 2 * bs2:
            a[bs2:2 * bs2] = 0  # an all-zero group
        q, s2 = nf4.double_quant(torch.from_numpy(a).cuda(), bs2)
        q_ref, s_ref = orc.double_quant(a, bs2)
        assert np.array_equal(q.cpu().numpy(), q_ref)
        assert np.array_equal(s2.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_double_quant_ties(nf4, orc):
    a = np.array([127.0, 62.5, 63.5, 0.5, 1.5, 2.5, 1.0, 0.25] * 40, np.float32)
    q, s2 = nf4.double_quant(torch.from_numpy(a).cuda(), 256)
    q_ref, s_ref = orc.double_quant(a, 256)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert q_ref[1] == 62 and q_ref[2] == 64


# ------------------------------------------------------------------ dequant


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_dequant_every_code_and_bf16_scale(nf4, orc, qt):
    """All 16 codes times every finite non-negative bf16 absmax (fp32 and bf16
    outputs, bit-exact), through the plain-absmax path."""
    a = (np.arange(0x7F80, dtype=np.uint32) << 16).view(np.float32)
    nb = a.size
    codes = (np.arange(nb * 64) * 7 + np.arange(nb * 64) // 64) % 16
    packed = ((codes[0::2] << 4) | codes[1::2]).astype(np.uint8)
    qs = nf4.QuantState(torch.from_numpy(packed).cuda(), torch.from_numpy(a).cuda(), None, None,
                        (nb * 64,), 64, qt, False)
    ref = dict(packed=packed, absmax=a)
    check_dequant(nf4, orc, qs, ref, 64, qt, False)


# ---------------------------------------------------------------- products


def _gemv_case(nf4, orc, w_cpu, x_cpu, bs, qt, dq, check_quantize=True):
    N, K = w_cpu.shape
    qs, ref = check_quant(nf4, orc, w_cpu, bs, qt, dq)
    w32_ref, wc16 = orc.dequantize(ref["packed"], N * K, bs, qt, **oracle_scales(ref, dq))
    x16 = to_u16(x_cpu)
    y_ref = orc.matmul_bf16(x16, wc16.reshape(N, K))
    xd = dev(x_cpu)
    y32 = nf4.gemv(xd, qs, torch.float32)
    y16 = nf4.gemv(xd, qs, torch.bfloat16)
    rel = check_product(y32, y16, y_ref, wc16.reshape(N, K), x16)
    assert torch.equal(nf4.gemv(xd, qs, torch.float32), y32), "GEMV is not deterministic"
    return rel


@pytest.mark.parametrize("cfg", [workloads.TINY, workloads.SQUARE_OUTLIERS], ids=lambda c: c.name)
def test_gemv_small_configs(nf4, orc, cfg):
    m = cfg.matrices[0]
    _gemv_case(nf4, orc, m.make(), cfg.activations(m.cols, 1), 64, "nf4", cfg.double_quant)


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
@pytest.mark.parametrize("which", [0, 1], ids=["up-11008x4096", "down-4096x11008"])
def test_gemv_mlp_config(nf4, orc, qt, which):
    """Batched decode M in {1, 4, 8, 16}: the oracle runs once on 16 rows and
    each M uses the leading rows."""
    m = workloads.MLP.matrices[which]
    w = m.make()
    N, K = w.shape
    qs, ref = check_quant(nf4, orc, w, 64, qt, True)
    _, wc16 = orc.dequantize(ref["packed"], N * K, 64, qt, **oracle_scales(ref, True))
    wc16 = wc16.reshape(N, K)
    x = workloads.MLP.activations(K, 16)
    x16 = to_u16(x)
    y_ref = orc.matmul_bf16(x16, wc16)
    for M in workloads.MLP.ms:
        xd = dev(x[:M])
        y32 = nf4.gemv(xd, qs, torch.float32)
        y16 = nf4.gemv(xd, qs, torch.bfloat16)
        check_product(y32, y16, y_ref[:M], wc16, x16[:M])


@pytest.mark.parametrize("bs", [32, 64, 128])
@pytest.mark.parametrize("dq", [False, True])
def test_gemv_ragged_shapes(nf4, orc, bs, dq):
    for (N, K, M) in [(1, bs, 1), (15, 2 * bs, 3), (17, 160 if bs == 32 else 5 * bs, 16),
                      (33, 4128 if bs == 32 else 33 * bs, 2), (100, 3 * bs, 7)]:
        w = workloads.normal_bf16((N, K), 0.02, N * 31 + K)
        x = workloads.normal_bf16((M, K), 1.0, N + K + M)
        _gemv_case(nf4, orc, w, x, bs, "nf4", dq)


@pytest.mark.parametrize("bs", [32, 64, 128, 256])
@pytest.mark.parametrize("dq", [False, True])
def test_gemv_single_row_long_k(nf4, orc, bs, dq):
    """M = 1 across row lengths that take one to four 4096-code slices per
    lane group, ragged last slices, an odd number of blocks per row (bs 32:
    a lane's two blocks can then straddle a double-quant group), the longest
    row the single-row kernel takes and one code block past it."""
    for i, K in enumerate([4096 + bs, 6144, 8192 + 3 * bs, 12288 + bs, 16384, 16384 + bs]):
        N = 45 + i
        w = workloads.normal_bf16((N, K), 0.02, 9100 + K + bs)
        x = workloads.normal_bf16((1, K), 1.0, 9200 + K)
        _gemv_case(nf4, orc, w, x, bs, "nf4", dq)


def test_gemv_grouped_m1_mixes_bs32_and_long_rows(nf4, orc):
    """A grouped M = 1 call with a blocksize-32 product (single-row kernel), a
    blocksize-64 product four slices long (single-row kernel, split into its
    own launch) and a blocksize-32 product four slices long (MFMA decode
    kernel): each equals its single call bit for bit and the oracle."""
    shapes = [(40, 8192, 32), (56, 16384, 64), (24, 16384, 32)]
    qss, xs, refs = [], [], []
    for i, (N, K, bs) in enumerate(shapes):
        w = workloads.normal_bf16((N, K), 0.02, 9500 + i)
        qs, ref = check_quant(nf4, orc, w, bs, "nf4", True)
        qss.append(qs)
        refs.append((ref, N, K, bs))
        xs.append(workloads.normal_bf16((1, K), 1.0, 9600 + i))
    ys = nf4.gemv_grouped([dev(x) for x in xs], qss, torch.float32)
    for i, (ref, N, K, bs) in enumerate(refs):
        y1 = nf4.gemv(dev(xs[i]), qss[i], torch.float32)
        assert torch.equal(ys[i], y1), f"product {i}: grouped differs from single"
        _, wc16 = orc.dequantize(ref["packed"], N * K, bs, "nf4", **oracle_scales(ref, True))
        x16 = to_u16(xs[i])
        y_ref = orc.matmul_bf16(x16, wc16.reshape(N, K))
        yy = y1.cpu().numpy().astype(np.float64)
        bound = PER_ELEM * np.linalg.norm(u16_to_f64(x16)) * np.linalg.norm(
            u16_to_f64(wc16.reshape(N, K)), axis=1)[None, :]
        assert np.all(np.abs(yy - y_ref) <= bound)
        assert np.linalg.norm(yy - y_ref) / np.linalg.norm(y_ref) <= REL_L2


@pytest.mark.parametrize("M", [1, 3])
def test_gemv_reads_no_activation_past_k(nf4, orc, M):
    """Rows whose length ends half-way through a lane's 64 codes (K % 64 == 32),
    with NaN bf16 values right after the activations in memory: nothing past
    x[:, K-1] may reach the sums."""
    for (N, K) in [(40, 160), (24, 4128)]:
        w = workloads.normal_bf16((N, K), 0.02, 5100 + K)
        x = workloads.normal_bf16((M, K), 1.0, 5200 + K + M)
        qs, ref = check_quant(nf4, orc, w, 32, "nf4", False)
        _, wc16 = orc.dequantize(ref["packed"], N * K, 32, "nf4", **oracle_scales(ref, False))
        y_ref = orc.matmul_bf16(to_u16(x), wc16.reshape(N, K))
        buf = torch.full((M * K + 4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
        buf[:M * K] = dev(x).reshape(-1)
        xd = buf[:M * K].view(M, K)
        y32 = nf4.gemv(xd, qs, torch.float32)
        assert torch.isfinite(y32).all(), "values past the activations were read"
        check_product(y32, None, y_ref, wc16.reshape(N, K), to_u16(x))


@pytest.mark.parametrize("dq", [False, True])
def test_gemv_batched_tile_counts(nf4, orc, dq):
    """Batched decode from a handful to thousands of 16-row tiles (more work
    items than workgroups, so each workgroup takes several in turn), with
    ragged rows and a ragged last 128-code step."""
    for (N, K, M) in [(2001, 1088, 16), (20000, 512, 2), (40000, 256, 5), (70007, 128, 16),
                      (100, 256, 3)]:
        w = workloads.normal_bf16((N, K), 0.02, 4200 + N + K)
        x = workloads.normal_bf16((M, K), 1.0, 4300 + N + M)
        _gemv_case(nf4, orc, w, x, 64, "nf4", dq)


@pytest.mark.parametrize("dq", [False, True])
def test_gemv_grouped_matches_single_and_oracle(nf4, orc, dq):
    """One grouped call over differently shaped products (three blocksizes,
    ragged rows, one row longer than the single-row kernel takes): each
    result is bitwise the single-product result and within tolerance of the
    oracle."""
    shapes = [(4096, 4096, 64), (1000, 512, 128), (33, 160, 32), (11008, 4096, 64), (16, 64, 64),
              (40, 16448, 64)]
    for M in (1, 3, 16):
        qss, xs, refs = [], [], []
        for i, (N, K, bs) in enumerate(shapes):
            w = workloads.normal_bf16((N, K), 0.02, 700 + i)
            x = workloads.normal_bf16((M, K), 1.0, 800 + i + M)
            qs, ref = check_quant(nf4, orc, w, bs, "nf4", dq)
            _, wc16 = orc.dequantize(ref["packed"], N * K, bs, "nf4", **oracle_scales(ref, dq))
            refs.append((orc.matmul_bf16(to_u16(x), wc16.reshape(N, K)), wc16.reshape(N, K),
                         to_u16(x)))
            qss.append(qs)
            xs.append(dev(x))
        ys = nf4.gemv_grouped(xs, qss, torch.float32)
        for y, x, qs, (y_ref, wc16, x16) in zip(ys, xs, qss, refs):
            assert torch.equal(y, nf4.gemv(x, qs, torch.float32))
            check_product(y, None, y_ref, wc16, x16)


def test_gemm_small_shapes(nf4, orc):
    for (M, N, K, bs, dq, qt) in [(1, 64, 64, 64, False, "nf4"), (5, 130, 256, 64, True, "nf4"),
                                  (128, 128, 128, 64, True, "fp4"), (130, 257, 96, 32, False, "nf4"),
                                  (300, 200, 512, 128, True, "nf4"), (64, 1, 64, 64, False, "fp4"),
                                  # double quant with more block scales per tile than the
                                  # kernel stages on chip (bs 32, long rows)
                                  (65, 230, 3072, 32, True, "nf4")]:
        w = workloads.normal_bf16((N, K), 0.02, M + N + K)
        x = workloads.normal_bf16((M, K), 1.0, M * N + K)
        qs, ref = check_quant(nf4, orc, w, bs, qt, dq)
        _, wc16 = orc.dequantize(ref["packed"], N * K, bs, qt, **oracle_scales(ref, dq))
        x16 = to_u16(x)
        y_ref = orc.matmul_bf16(x16, wc16.reshape(N, K))
        xd = dev(x)
        y32 = nf4.gemm(xd, qs, torch.float32)
        y16 = nf4.gemm(xd, qs, torch.bfloat16)
        check_product(y32, y16, y_ref, wc16.reshape(N, K), x16)


def test_gemm_prefill_config(nf4, orc):
    """Full prefill shape 2048 x 4096 x 14336, NF4 bs64 + double quant:
    quantize bit-exact; 4096 sampled outputs against the fp64 oracle; all
    outputs: bf16 == RNE(fp32), determinism, nf4_linear with a workspace (the
    weight dequantized once) bitwise nf4_gemm, and the first 16 rows against
    the (separately parity-tested) GEMV kernel."""
    cfg = workloads.PREFILL
    m = cfg.matrices[0]
    w = m.make()
    N, K = w.shape
    M = cfg.ms[0]
    qs, ref = check_quant(nf4, orc, w, 64, "nf4", True)
    _, wc16 = orc.dequantize(ref["packed"], N * K, 64, "nf4", **oracle_scales(ref, True))
    wc16 = wc16.reshape(N, K)
    x = cfg.activations(K, M)
    x16 = to_u16(x)
    xd = dev(x)
    y32 = nf4.gemm(xd, qs, torch.float32)
    y16 = nf4.gemm(xd, qs, torch.bfloat16)
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(nf4.gemm(xd, qs, torch.float32), y32), "GEMM is not deterministic"
    # nf4_linear with a workspace: the weight dequantized once, the same bits
    assert torch.equal(nf4.linear(xd, qs, out_dtype=torch.float32), y32)
    rng = np.random.default_rng(5)
    ms = rng.integers(0, M, 4096)
    ns = rng.integers(0, N, 4096)
    ms[:4] = [0, M - 1, 0, M - 1]
    ns[:4] = [0, 0, N - 1, N - 1]
    ys_ref = orc.matmul_bf16_sampled(x16, wc16, ms, ns)
    ys = y32.cpu().numpy().astype(np.float64)[ms, ns]
    bound = PER_ELEM * np.linalg.norm(u16_to_f64(wc16)[ns], axis=1) * np.linalg.norm(
        u16_to_f64(x16)[ms], axis=1)
    assert np.all(np.abs(ys - ys_ref) <= bound)
    assert np.linalg.norm(ys - ys_ref) / np.linalg.norm(ys_ref) <= REL_L2
    yv = nf4.gemv(xd[:16], qs, torch.float32)
    diff = (yv - y32[:16]).abs()
    assert torch.all(diff <= 1e-4 * (y32[:16].abs() + yv.abs()) + 1e-3)


def test_gemm_prefill_full_output(nf4, orc):
    """Every output of the full prefill GEMM (2048 x 4096 x 14336, NF4 bs64 +
    double quant, fp32 out) against the fp64 oracle, computed by the oracle's
    decode product split over host threads (bitwise its single-threaded
    result): each element within 1e-3 ||w_row|| ||x_row||, rel-L2 <= 1e-4."""
    import os

    cfg = workloads.PREFILL
    m = cfg.matrices[0]
    w = m.make()
    N, K = w.shape
    M = cfg.ms[0]
    qs, ref = check_quant(nf4, orc, w, 64, "nf4", True)
    x = cfg.activations(K, M)
    x16 = to_u16(x)
    y = nf4.gemm(dev(x), qs, torch.float32).cpu().numpy().astype(np.float64)
    threads = max(1, min(16, os.cpu_count() or 1))
    y_ref = orc.gemv_quantized_threads(x16, ref["packed"], N, K, threads, 64, "nf4",
                                       absmax_q=ref["absmax_q"], absmax_scale=ref["absmax_scale"])
    _, wc16 = orc.dequantize(ref["packed"], N * K, 64, "nf4", **oracle_scales(ref, True))
    wn = np.linalg.norm(u16_to_f64(wc16.reshape(N, K)), axis=1)
    xn = np.linalg.norm(u16_to_f64(x16), axis=1)
    err = np.abs(y - y_ref)
    assert np.all(err <= PER_ELEM * xn[:, None] * wn[None, :]), \
        f"max err / bound {np.max(err / (PER_ELEM * xn[:, None] * wn[None, :])):.3e}"
    assert np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref) <= REL_L2


def test_decode_k_5120_many_rows_grouped(nf4, orc):
    """K in 4097..6144 (three 128-code chunks per wave in the register-resident
    decode kernel) with enough rows that two-tile items would be counted: a
    grouped call of two [13824, 5120] products at M = 4 covers every row
    (sampled rows against the oracle, all rows against the single calls)."""
    K, N = 5120, 13824
    qss, refs, ws = [], [], []
    for j in range(2):
        w = workloads.normal_bf16((N, K), 0.02, 6100 + j)
        qs, ref = check_quant(nf4, orc, w, 64, "nf4", True)
        qss.append(qs)
        refs.append(ref)
    x = workloads.normal_bf16((4, K), 1.0, 6200)
    x16 = to_u16(x)
    xd = dev(x)
    outs = [torch.full((4, N), float("nan"), device="cuda") for _ in range(2)]
    ys = nf4.gemv_grouped([xd, xd], qss, torch.float32, outs=outs)
    rng = np.random.default_rng(11)
    rows = np.concatenate([[0, N - 1, N // 2], rng.integers(0, N, 61)])
    for j in range(2):
        y1 = nf4.gemv(xd, qss[j], torch.float32)
        assert torch.equal(ys[j], y1), "grouped differs from single"
        _, wc16 = orc.dequantize(refs[j]["packed"], N * K, 64, "nf4", **oracle_scales(refs[j], True))
        wsel = wc16.reshape(N, K)[rows]
        y_ref = orc.matmul_bf16(x16, np.ascontiguousarray(wsel))
        yy = ys[j].cpu().numpy().astype(np.float64)[:, rows]
        bound = PER_ELEM * np.linalg.norm(u16_to_f64(x16), axis=1)[:, None] * \
            np.linalg.norm(u16_to_f64(wsel), axis=1)[None, :]
        assert np.all(np.abs(yy - y_ref) <= bound)
        assert bool(torch.isfinite(ys[j]).all()), "rows left unwritten"


@pytest.mark.parametrize("bs", [64, 128, 256])
def test_stack7b_sampled_matrices(nf4, orc, bs):
    """7B-shaped stack at each blocksize: first and last layer's q-shaped and
    mlp-shaped matrices, quantize + double quant + dequant bit-exact and the
    M=1 GEMV within tolerance."""
    mats = workloads.STACK_7B.matrices
    for mat in (mats[0], mats[4], mats[-1]):
        w = mat.make()
        N, K = w.shape
        qs, ref = check_quant(nf4, orc, w, bs, "nf4", True)
        wc16 = check_dequant(nf4, orc, qs, ref, bs, "nf4", True).reshape(N, K)
        x = workloads.normal_bf16((1, K), 1.0, mat.seed + 1000)
        x16 = to_u16(x)
        y_ref = orc.matmul_bf16(x16, wc16)
        y32 = nf4.gemv(dev(x), qs, torch.float32)
        check_product(y32, None, y_ref, wc16, x16)


# ------------------------------------------------------------ linear + bias


@pytest.mark.parametrize("M,N,K,bs,dq", [
    (1, 1000, 512, 64, True),     # single-row kernel
    (1, 300, 20480, 64, True),    # K > 16384: the K-split kernel at M = 1
    (4, 1000, 512, 64, True),     # x in registers
    (4, 130, 8192, 128, False),   # K > 6144: the K-split kernel
    (16, 257, 1024, 64, True),
    (17, 300, 512, 64, True),     # two 16-row M tiles
    (64, 1000, 512, 32, False),   # the largest decode batch
    (65, 300, 512, 64, True),     # past the decode range: the prefill GEMM
    (130, 200, 256, 32, False),
])
def test_linear_bias_matches_oracle(nf4, orc, M, N, K, bs, dq):
    """nf4_linear with a bf16 bias against the oracle's linear layer, each path
    of the dispatch; without a bias it is bitwise nf4_gemv / nf4_gemm, and with
    one it is bitwise RN_fp32(that result + bias)."""
    w = workloads.normal_bf16((N, K), 0.02, 7 * M + N + K)
    x = workloads.normal_bf16((M, K), 1.0, 11 * M + K)
    b = workloads.normal_bf16((N,), 0.5, 13 * N + M)
    qs, ref = check_quant(nf4, orc, w, bs, "nf4", dq)
    _, wc16 = orc.dequantize(ref["packed"], N * K, bs, "nf4", **oracle_scales(ref, dq))
    x16, b16 = to_u16(x), to_u16(b)
    y_ref = orc.linear_bf16(x16, wc16.reshape(N, K), b16)
    xd, bd = dev(x), dev(b)
    y32 = nf4.linear(xd, qs, bd, torch.float32)
    y16 = nf4.linear(xd, qs, bd, torch.bfloat16)
    check_product(y32, y16, y_ref, wc16.reshape(N, K), x16, b16)
    y_nb = nf4.linear(xd, qs, None, torch.float32)
    direct = nf4.gemv(xd, qs, torch.float32) if M <= 64 else nf4.gemm(xd, qs, torch.float32)
    assert torch.equal(y_nb, direct), "without a bias, nf4_linear differs from the direct call"
    assert torch.equal(y32, y_nb + bd.float()[None, :]), "the bias is not one fp32 add"
    assert torch.equal(nf4.linear(xd, qs, bd, torch.float32), y32), "not deterministic"


def test_linear_rejects_misaligned_bias(nf4):
    w = workloads.normal_bf16((64, 64), 0.02, 5)
    qs = nf4.quantize(dev(w), 64, "nf4", double_quant=False)
    x = dev(workloads.normal_bf16((1, 64), 1.0, 6))
    y = torch.empty((1, 64), dtype=torch.float32, device="cuda")
    raw = torch.zeros(65, dtype=torch.uint8, device="cuda")
    d = qs.desc()
    import ctypes
    st = nf4.lib().nf4_linear(ctypes.c_void_p(x.data_ptr()), 1, ctypes.byref(d), 64, 64,
                              ctypes.c_void_p(raw.data_ptr() + 1), 0, 1,
                              ctypes.c_void_p(y.data_ptr()), None)
    assert st == 3, f"status {st}, expected NF4_ERR_MISALIGNED"


# ----------------------------------------------- descriptor scale pointers


@pytest.mark.parametrize("M", [17, 64])
def test_products_read_only_the_scales_the_flag_selects(nf4, orc, M):
    """A descriptor may carry stale pointers in the scale fields its
    double-quant flag does not select (the header: absmax is read when
    double_quant == 0, absmax_q / absmax_scale when it is 1). nf4_gemm and
    nf4_linear must give bitwise the result of the descriptor with those
    fields NULL, for both flag values, and match the oracle."""
    import ctypes

    N, K, bs = 300, 1024, 64
    w = workloads.normal_bf16((N, K), 0.02, 4400 + M)
    x = workloads.normal_bf16((M, K), 1.0, 4500 + M)
    xd = dev(x)
    x16 = to_u16(x)
    nb = N * K // bs
    g = torch.Generator(device="cuda").manual_seed(M)
    junk_q = torch.randint(-128, 128, (nb,), dtype=torch.int8, device="cuda", generator=g)
    junk_s = torch.rand((nb + 255) // 256, device="cuda", generator=g) * 100
    junk_a = torch.rand(nb, device="cuda", generator=g) * 100
    for dq in (False, True):
        qs, ref = check_quant(nf4, orc, w, bs, "nf4", dq)
        _, wc16 = orc.dequantize(ref["packed"], N * K, bs, "nf4", **oracle_scales(ref, dq))
        y_ref = orc.matmul_bf16(x16, wc16.reshape(N, K))
        clean = qs.desc()
        dirty = qs.desc()
        if dq:
            clean.absmax = None
            dirty.absmax = junk_a.data_ptr()
        else:
            clean.absmax_q = clean.absmax_scale = None
            dirty.absmax_q, dirty.absmax_scale = junk_q.data_ptr(), junk_s.data_ptr()
        outs = {}
        for name, d in (("clean", clean), ("dirty", dirty)):
            for fn in ("nf4_gemm", "nf4_linear"):
                y = torch.empty((M, N), dtype=torch.float32, device="cuda")
                args = [ctypes.c_void_p(xd.data_ptr()), M, ctypes.byref(d), N, K]
                if fn == "nf4_linear":
                    args.append(None)
                args += [nf4.DTYPE_BF16, nf4.DTYPE_FP32, ctypes.c_void_p(y.data_ptr()), None]
                assert getattr(nf4.lib(), fn)(*args) == 0, (fn, name, dq)
                outs[(name, fn)] = y
        torch.cuda.synchronize()
        for fn in ("nf4_gemm", "nf4_linear"):
            assert torch.equal(outs[("clean", fn)], outs[("dirty", fn)]), (fn, dq)
            check_product(outs[("dirty", fn)], None, y_ref, wc16.reshape(N, K), x16)


# ------------------------------------------- a 7B layer, grouped, batched


@pytest.mark.parametrize("dq", [False, True])
def test_gemv_grouped_7b_layer_batched(nf4, orc, dq):
    """The seven products of one 7B-shaped layer (4 x [4096, 4096],
    3 x [11008, 4096], NF4 bs 64) in one grouped call at M = 4 and 16: each
    output bitwise equals the product launched alone and is within tolerance
    of the oracle. Grouped, the launch holds enough rows for the kernels'
    large-launch work items, which single products do not reach."""
    shapes = [(4096, 4096)] * 4 + [(11008, 4096)] * 3
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert sum(n for n, _ in shapes) // 32 >= 4 * cu, "the layer no longer reaches big items"
    qss, refs = [], []
    for i, (N, K) in enumerate(shapes):
        w = workloads.normal_bf16((N, K), 0.02, 8800 + i)
        qs, ref = check_quant(nf4, orc, w, 64, "nf4", dq)
        qss.append(qs)
        refs.append(ref)
    x = workloads.normal_bf16((16, 4096), 1.0, 8899)
    x16 = to_u16(x)
    for M in (4, 16):
        xd = dev(x[:M])
        ys = nf4.gemv_grouped([xd] * 7, qss, torch.float32)
        for i, ((N, K), qs, ref, y) in enumerate(zip(shapes, qss, refs, ys)):
            assert torch.equal(y, nf4.gemv(xd, qs, torch.float32)), (M, i)
            if i in (0, 4):  # one product of each shape against the oracle
                y_ref = orc.gemv_quantized(x16[:M], ref["packed"], N, K, 64, "nf4",
                                           **oracle_scales(ref, dq))
                _, wc16 = orc.dequantize(ref["packed"], N * K, 64, "nf4", **oracle_scales(ref, dq))
                check_product(y, None, y_ref, wc16.reshape(N, K), x16[:M])
