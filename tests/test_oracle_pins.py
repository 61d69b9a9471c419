"""Pins for the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
NF4 page prints, library routines (statistics.NormalDist, numpy float32/float64
arithmetic and BLAS, torch's bf16 conversion), exact rational brute force,
hand-worked examples and invariants of the method. A plausible slip in the
oracle (wrong delta or 7/8 split, a sign, a nibble order, a tie rule, a
transposed operand, a dropped scale) fails at least one of them.
"""
import os
from fractions import Fraction
from statistics import NormalDist

import numpy as np
import pytest
import torch

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DELTA = 929.0 / 960.0


def f32(v):
    return np.float32(v)


def bits(v):
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])


# --------------------------------------------------------------- codebook


def test_nf4_values_printed_on_page(orc):
    """NF4 page, table 数学原理对比, row 数值表示."""
    cb = orc.codebook("nf4")
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "nf4_page_values.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 5
    for code, val, tol in rows:
        assert abs(float(cb[int(code)]) - float(val)) <= float(tol), (code, cb[int(code)], val)


def test_nf4_structure(orc):
    """Sorted, inside [-1, 1], exact 0 (row 零点: no zero-point, 0 is a code),
    7 negative and 8 positive values, extremes exactly -1 and +1."""
    cb = orc.codebook("nf4").astype(np.float64)
    assert np.all(np.diff(cb) > 0)
    assert cb[0] == -1.0 and cb[15] == 1.0 and cb[7] == 0.0
    assert np.sum(cb < 0) == 7 and np.sum(cb > 0) == 8
    assert np.all(np.abs(cb) <= 1.0)


def test_norm_ppf_matches_library():
    """The oracle's bisection quantile agrees with CPython's NormalDist.inv_cdf
    (a different algorithm) to a few ulp over the range the codebook uses."""
    import oracle

    nd = NormalDist()
    for p in np.concatenate([np.linspace(0.5, 0.999, 301), 1 - np.logspace(-12, -3, 50),
                             np.linspace(1e-6, 0.5, 101)]):
        z0, z1 = oracle.norm_ppf(p), nd.inv_cdf(p)
        assert abs(z0 - z1) <= 4e-15 * max(1.0, abs(z1)), (p, z0, z1)


def test_nf4_levels_are_normal_quantiles(orc):
    """Forward check with the library CDF: Phi(c_j * Phi^-1(delta)) lands on the
    equally spaced probability levels, 8 steps above 1/2 and 7 below."""
    cb = orc.codebook("nf4").astype(np.float64)
    nd = NormalDist()
    zmax = nd.inv_cdf(DELTA)
    for j in range(1, 9):
        assert abs(nd.cdf(cb[7 + j] * zmax) - (0.5 + (DELTA - 0.5) * j / 8)) < 2e-8
    for j in range(1, 8):
        assert abs(nd.cdf(-cb[7 - j] * zmax) - (0.5 + (DELTA - 0.5) * j / 7)) < 2e-8


def test_nf4_fp32_rounding_is_robust(orc):
    """Every fp64 code value sits far from an fp32 rounding boundary, so any
    quantile routine accurate to 1e-12 gives the same fp32 table."""
    nd = NormalDist()
    zmax = nd.inv_cdf(DELTA)
    vals = [-nd.inv_cdf(0.5 + (DELTA - 0.5) * j / 7) / zmax for j in range(7, 0, -1)]
    vals += [0.0] + [nd.inv_cdf(0.5 + (DELTA - 0.5) * j / 8) / zmax for j in range(1, 9)]
    cb = orc.codebook("nf4")
    for v, c in zip(vals, cb):
        lo = np.nextafter(np.float32(v), np.float32(-2))
        hi = np.nextafter(np.float32(v), np.float32(2))
        assert np.float32(v) == c
        if v != 0:
            margin = min(abs(v - (float(lo) + float(np.float32(v))) / 2),
                         abs(v - (float(hi) + float(np.float32(v))) / 2))
            assert margin > 1e-12 * abs(v)


def test_fp4_is_e2m1_over_6(orc):
    """NF4 page, notes 补充说明: fp4 is an E2M1-like float. Magnitudes x 6 are the
    E2M1 value set; bit 3 is the sign; magnitude grows with the low 3 bits."""
    cb = orc.codebook("fp4").astype(np.float64)
    mags = sorted(set(np.round(np.abs(cb) * 6, 6)))  # fp32(k/12) * 6 is k/2 to ~1e-7
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for nib in range(16):
        assert np.float32(cb[nib]) == np.float32(abs(cb[nib & 7]) * (-1 if nib & 8 else 1))
    assert np.all(np.diff(cb[:8]) > 0)
    assert cb[0] == 0.0 and np.signbit(cb[0]) == False  # noqa: E712
    assert cb[8] == 0.0 and np.signbit(cb[8])
    assert cb[7] == 1.0 and cb[15] == -1.0
    # fp32 roundings of k/12
    for nib, k in [(1, 1), (2, 2), (4, 4), (6, 8)]:
        assert cb[nib] == np.float32(k / 12.0)


# ---------------------------------------------------------- code function


def _sorted_candidates(orc, qt):
    cb = orc.codebook(qt)
    codes = [c for c in range(16) if not (qt == "fp4" and c == 8)]
    codes.sort(key=lambda c: float(cb[c]))
    return cb, codes


def _brute_nearest(s, cb, codes):
    """Exact rational nearest; ties go to the smaller code value."""
    fs = Fraction(float(s))
    best, bd = None, None
    for c in codes:
        d = abs(fs - Fraction(float(cb[c])))
        if bd is None or d < bd:
            best, bd = c, d
    return best


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_nearest_code_brute_force(orc, qt):
    """NF4 page, row 量化目标: the code minimises the squared error. Exact
    rational brute force on random values and on every midpoint +-2 ulp."""
    cb, codes = _sorted_candidates(orc, qt)
    rng = np.random.default_rng(7)
    probes = list(rng.uniform(-1, 1, 400).astype(np.float32))
    for a, b in zip(codes[:-1], codes[1:]):
        mid = np.float32((float(cb[a]) + float(cb[b])) / 2)
        v = mid
        for _ in range(3):
            v = np.nextafter(v, np.float32(-2))
        for _ in range(5):
            probes.append(v)
            v = np.nextafter(v, np.float32(2))
    probes += [np.float32(0.0), np.float32(-0.0), np.float32(1.0), np.float32(-1.0), np.float32(1e-30)]
    for s in probes:
        assert orc.nearest_code(float(s), qt) == _brute_nearest(s, cb, codes), s


def _rd_thresholds(cb, codes):
    """Largest fp32 not above each exact midpoint (computed with Fractions)."""
    out = []
    for a, b in zip(codes[:-1], codes[1:]):
        m = (Fraction(float(cb[a])) + Fraction(float(cb[b]))) / 2
        t = np.float32(float(m))
        if Fraction(float(t)) > m:
            t = np.nextafter(t, np.float32(-2))
        out.append(t)
    return np.array(out, dtype=np.float32)


def _all_bf16_classes():
    """For a in [1, 2) (all 128 bf16 significands) and every finite bf16 x with
    |x| <= a: RN(x / a) depends only on the significands and the exponent gap,
    so these classes cover every normal (x, a) pair. Laid out as blocks of 64
    whose first element is a, so the block absmax is a."""
    a_bits = (0x3F80 | np.arange(128)).astype(np.uint16)
    allx = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    xf = (allx.astype(np.uint32) << 16).view(np.float32)
    blocks = []
    for ab in a_bits:
        af = (np.array([ab], np.uint32) << 16).view(np.float32)[0]
        xs = allx[np.isfinite(xf) & (np.abs(xf) <= af)]
        pad = (-len(xs)) % 63
        xs = np.concatenate([xs, np.zeros(pad, np.uint16)]).reshape(-1, 63)
        blk = np.concatenate([np.full((xs.shape[0], 1), ab, np.uint16), xs], axis=1)
        blocks.append(blk)
    return np.concatenate(blocks).reshape(-1)


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_code_function_all_bf16_classes(orc, qt):
    """Exhaustive: the oracle's quantize agrees with an independent threshold
    formulation (numpy IEEE float32 division, then count of round-down fp32
    midpoints strictly below s) on every bf16 (x, a) class."""
    w = _all_bf16_classes()
    packed, absmax = orc.quantize(w, 64, qt)
    cb, codes = _sorted_candidates(orc, qt)
    thr = _rd_thresholds(cb, codes)
    xf = (w.astype(np.uint32) << 16).view(np.float32)
    a = np.repeat(absmax, 64)[: w.size]
    with np.errstate(invalid="ignore"):
        s = np.where(a == 0, np.float32(0), xf / a).astype(np.float32)
    rank = np.searchsorted(thr, s, side="left")  # number of thresholds < s
    expect = np.array(codes)[rank]
    assert np.array_equal(_codes(packed, w.size), expect)


# ---------------------------------------------------------------- quantize


def _codes(packed, n):
    c = np.empty(2 * packed.size, np.int64)
    c[0::2] = packed >> 4
    c[1::2] = packed & 15
    return c[:n]


def test_quantize_worked_example(orc):
    """Hand-worked from the codebook: with a = 1, s = x; the nearest NF4 values
    are 1 -> 15, -0.5 -> -0.525 (2), 0.25 -> 0.2461 (10), 0 -> 7, -1 -> 0,
    0.6992 -> 0.7230 (14), 0.1001 -> 0.0796 (8), -0.0898 -> -0.0910 (6); FP4:
    1 -> 7, -0.5 -> D, 0.25 -> 3, 0 -> 0, -1 -> F, 0.6992 -> 2/3 (6),
    0.1001 -> 1/12 (1), -0.0898 -> -1/12 (9). Element 2i is the high nibble."""
    x = workloads.to_u16(torch.tensor([1.0, -0.5, 0.25, 0.0, -1.0, 0.7, 0.1, -0.09]).to(torch.bfloat16))
    p, a = orc.quantize(x, 64, "nf4")
    assert list(_codes(p, 8)) == [15, 2, 10, 7, 0, 14, 8, 6]
    assert bytes(p) == bytes([0xF2, 0xA7, 0x0E, 0x86])
    assert a.tolist() == [1.0]
    p, a = orc.quantize(x, 64, "fp4")
    assert list(_codes(p, 8)) == [7, 13, 3, 0, 15, 6, 1, 9]
    assert bytes(p) == bytes([0x7D, 0x30, 0xF6, 0x19])


def test_quantize_odd_length_pad_nibble(orc):
    x = workloads.to_u16(torch.tensor([0.5, -0.25, 1.0]).to(torch.bfloat16))
    p, a = orc.quantize(x, 64, "nf4")
    assert p.size == 2 and (p[1] & 15) == 0 and (p[1] >> 4) == 15


@pytest.mark.parametrize("bs", [32, 64, 128, 256, 4096])
def test_absmax_and_extremes(orc, bs):
    """Per-block absmax equals numpy's max |x| over the block's real elements
    (partial last block included); the element carrying it maps to +-1."""
    n = 3 * bs + bs // 2 + 3
    w = workloads.to_u16(workloads.normal_bf16((n,), 0.02, 11))
    for qt, hi_code, lo_code in [("nf4", 15, 0), ("fp4", 7, 15)]:
        p, a = orc.quantize(w, bs, qt)
        xf = (w.astype(np.uint32) << 16).view(np.float32)
        nb = -(-n // bs)
        assert a.size == nb
        codes = _codes(p, n)
        for b in range(nb):
            blk = xf[b * bs:(b + 1) * bs]
            assert a[b] == np.max(np.abs(blk))
            i = int(np.argmax(np.abs(blk)))
            assert codes[b * bs + i] == (hi_code if blk[i] > 0 else lo_code)


def test_zero_block(orc):
    w = np.zeros(128, np.uint16)
    w[64:] = workloads.to_u16(workloads.normal_bf16((64,), 1.0, 3))
    p, a = orc.quantize(w, 64, "nf4")
    assert a[0] == 0 and np.all(_codes(p, 128)[:64] == 7)
    p, a = orc.quantize(w, 64, "fp4")
    assert np.all(_codes(p, 128)[:64] == 0)


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_monotone_and_error_bound(orc, qt):
    """Within a block the code value is non-decreasing in x, and the
    reconstruction error is at most half the widest code gap times a (plus
    rounding)."""
    cb = orc.codebook(qt).astype(np.float64)
    n = 64 * 50
    w = workloads.to_u16(workloads.normal_bf16((n,), 0.02, 5))
    p, a = orc.quantize(w, 64, qt)
    xf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    v = cb[_codes(p, n)]
    svals = np.sort(np.unique(cb))
    gap = np.max(np.diff(svals))
    for b in range(50):
        sl = slice(b * 64, (b + 1) * 64)
        order = np.argsort(xf[sl], kind="stable")
        assert np.all(np.diff(v[sl][order]) >= 0)
        err = np.abs(xf[sl] - v[sl] * a[b])
        assert np.all(err <= a[b] * (gap / 2 + 1e-6))


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_quantize_dequantize_idempotent(orc, qt):
    """Re-quantizing the bf16 dequantized tensor returns the same codes and the
    same absmax (no double quant): codewords are fixed points."""
    n = 64 * 40 + 17
    w = workloads.to_u16(workloads.normal_bf16((n,), 0.02, 9))
    p, a = orc.quantize(w, 64, qt)
    _, w16 = orc.dequantize(p, n, 64, qt, absmax=a)
    p2, a2 = orc.quantize(w16, 64, qt)
    assert np.array_equal(a, a2)
    c1, c2 = _codes(p, n), _codes(p2, n)
    if qt == "fp4":  # -0 and +0 are the same value
        c1 = np.where(c1 == 8, 0, c1)
    assert np.array_equal(c1, c2)


# ------------------------------------------------------------ double quant


def test_double_quant_worked_example(orc):
    """Hand-worked: s2 = RN(1/127); a/s2 -> 127, 63.5..., 31.75, 0, 95.25, 15.875."""
    q, s2 = orc.double_quant(np.array([1.0, 0.5, 0.25, 0.0, 0.75, 0.125], np.float32), 256)
    assert q.tolist() == [127, 64, 32, 0, 95, 16]
    assert s2[0] == f32(1) / f32(127)
    assert bits(s2[0]) == 0x3C010204


def test_double_quant_ties_to_even(orc):
    """m = 127 gives s2 = 1 exactly, so a/s2 = a: 62.5 -> 62, 63.5 -> 64,
    0.5 -> 0, 1.5 -> 2 (round half to even)."""
    q, s2 = orc.double_quant(np.array([127.0, 62.5, 63.5, 0.5, 1.5, 2.5], np.float32), 256)
    assert s2[0] == 1.0
    assert q.tolist() == [127, 62, 64, 0, 2, 2]


def test_double_quant_groups_and_invariants(orc):
    nb = 256 * 5 + 77
    rng = np.random.default_rng(4)
    a = (np.abs(rng.standard_normal(nb)) * 0.05).astype(np.float32)
    a[256:512] = 0.0  # an all-zero group
    q, s2 = orc.double_quant(a, 256)
    assert s2.size == 6
    assert s2[1] == 0 and np.all(q[256:512] == 0)
    for g in range(6):
        blk = a[g * 256:(g + 1) * 256]
        qb = q[g * 256:(g + 1) * 256].astype(np.int64)
        assert np.all((qb >= 0) & (qb <= 127))
        if blk.max() > 0:
            assert s2[g] == f32(blk.max()) / f32(127)
            assert qb[int(np.argmax(blk))] == 127
            ap = (qb.astype(np.float32) * s2[g]).astype(np.float64)
            assert np.all(np.abs(ap - blk) <= s2[g] / 2 * (1 + 2 ** -14))
            # numpy float32 IEEE division + rint (round half even)
            assert np.array_equal(qb, np.rint((blk / s2[g]).astype(np.float32)).astype(np.int64))


# ----------------------------------------------------------------- dequant


def test_dequant_products_and_bf16(orc):
    """w = RN(c * a') matches numpy float32 multiplication for all 16 codes;
    the bf16 compute dtype matches torch's fp32 -> bf16 conversion."""
    for qt in ["nf4", "fp4"]:
        cb = orc.codebook(qt)
        rng = np.random.default_rng(1)
        a = np.concatenate([np.abs(rng.standard_normal(30)).astype(np.float32) * 0.07,
                            np.array([1.0, 2.0 ** -130, 3.0e38], np.float32)])
        nb = a.size
        codes = np.tile(np.arange(16), nb * 4)[: nb * 64]
        packed = ((codes[0::2] << 4) | codes[1::2]).astype(np.uint8)
        w32, w16 = orc.dequantize(packed, nb * 64, 64, qt, absmax=a)
        expect = (cb[codes] * np.repeat(a, 64)).astype(np.float32)
        assert np.array_equal(w32.view(np.uint32), expect.view(np.uint32))
        t16 = workloads.to_u16(torch.from_numpy(expect).to(torch.bfloat16))
        assert np.array_equal(w16, t16)


def test_dequant_with_double_quant_scale(orc):
    n = 64 * 300
    w = workloads.to_u16(workloads.normal_bf16((n,), 0.02, 12))
    p, a = orc.quantize(w, 64, "nf4")
    q, s2 = orc.double_quant(a, 256)
    w32, _ = orc.dequantize(p, n, 64, "nf4", absmax_q=q, absmax_scale=s2)
    cb = orc.codebook("nf4")
    ap = (q.astype(np.float32) * np.repeat(s2, 256)[: a.size]).astype(np.float32)
    expect = (cb[_codes(p, n)] * np.repeat(ap, 64)).astype(np.float32)
    assert np.array_equal(w32.view(np.uint32), expect.view(np.uint32))


# ------------------------------------------------------------------ matmul


def test_matmul_matches_blas(orc):
    """fp64 sums agree with numpy float64 BLAS on non-square shapes (a
    transposed operand would not even have matching shapes)."""
    M, N, K = 3, 37, 192
    x = workloads.to_u16(workloads.normal_bf16((M, K), 1.0, 21))
    wc = workloads.to_u16(workloads.normal_bf16((N, K), 0.02, 22))
    y = orc.matmul_bf16(x, wc)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wf = (wc.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = xf @ wf.T
    assert y.shape == (M, N)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    ms, ns = np.array([0, 2, 1]), np.array([36, 0, 5])
    ys = orc.matmul_bf16_sampled(x, wc, ms, ns)
    assert np.allclose(ys, ref[ms, ns], rtol=1e-12, atol=0)


@pytest.mark.parametrize("dq", [False, True])
def test_gemv_quantized_equals_dequant_then_matmul(orc, dq):
    N, K, M = 24, 256, 2
    w = workloads.to_u16(workloads.normal_bf16((N, K), 0.02, 31))
    x = workloads.to_u16(workloads.normal_bf16((M, K), 1.0, 32))
    p, a = orc.quantize(w, 64, "nf4")
    kw = dict(absmax=a)
    if dq:
        q, s2 = orc.double_quant(a, 256)
        kw = dict(absmax_q=q, absmax_scale=s2)
    _, w16 = orc.dequantize(p, N * K, 64, "nf4", **kw)
    y = orc.gemv_quantized(x, p, N, K, 64, "nf4", **kw)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wf = (w16.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(N, K)
    ref = xf @ wf.T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_7b_storage_accounting():
    """NF4 page, intro: a 7B model in NF4 loads in about 3.5-4 GB. The linear
    weights of the 7B-shaped stack with double quant must fit below that."""
    n = sum(m.rows * m.cols for m in workloads.STACK_7B.matrices)
    assert n == 6_476_005_376
    for bs, expect_gb in [(64, 3.341), (128, 3.289), (256, 3.264)]:
        nb = -(-n // bs)
        total = -(-n // 2) + nb + 4 * (-(-nb // 256))
        assert abs(total / 1e9 - expect_gb) < 0.002
        assert 3.0 < total / 1e9 < 4.0


def test_linear_bias_hand_example(orc):
    """A worked example by hand: x = [[1, 2]], W = [[1, 1], [2, -1]], bias =
    [0.5, -3] -> y = [[1 + 2 + 0.5, 2 - 2 - 3]] = [[3.5, -3]]; and a zero x
    gives the bias itself in every row (every value here is exact in bf16)."""
    bf = lambda v: np.array([orc.f32_to_bf16(float(t)) for t in np.ravel(v)], dtype=np.uint16).reshape(
        np.shape(v))
    x = bf([[1.0, 2.0]])
    w = bf([[1.0, 1.0], [2.0, -1.0]])
    b = bf([0.5, -3.0])
    assert np.array_equal(orc.linear_bf16(x, w, b), np.array([[3.5, -3.0]]))
    assert np.array_equal(orc.linear_bf16(x, w, None), np.array([[3.0, 0.0]]))
    z = bf(np.zeros((3, 2)))
    assert np.array_equal(orc.linear_bf16(z, w, b), np.array([[0.5, -3.0]] * 3))


def test_oracle_builds_itself_when_library_missing(tmp_path):
    """A copy of oracle/ without its compiled library: the first call builds
    it (gcc) and computes the same codes as the regular build."""
    import shutil
    import subprocess
    import sys

    src = os.path.join(ROOT, "oracle")
    dst = tmp_path / "oracle"
    dst.mkdir()
    for name in os.listdir(src):
        if name.endswith((".py", ".c")):
            shutil.copy(os.path.join(src, name), dst / name)
    assert not (dst / "libnf4_oracle.so").exists()
    code = ("import numpy as np, oracle\n"
            "w = np.array([0x3f80, 0xbf00, 0x3e80, 0, 0xbf80, 0x3f33, 0x3dcd, 0xbdb8], np.uint16)\n"
            "p, a = oracle.quantize(w, 64, 'nf4')\n"
            "print(bytes(p).hex(), float(a[0]))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=str(tmp_path), capture_output=True,
                       text=True, env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode == 0, r.stderr
    assert (dst / "libnf4_oracle.so").exists()
    assert r.stdout.split() == ["f2a70e86", "1.0"]


# ----------------------------------------------------- fp16 and fp32 types


def test_fp16_decode_all_patterns(orc):
    """Every finite fp16 bit pattern decodes to numpy's float16 value."""
    h = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float32)
    fin = np.isfinite(ref)
    got = orc.convert(h, "fp16", "fp32")
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))


def test_fp16_rounding_matches_numpy(orc):
    """fp32 -> fp16 round-to-nearest-even against numpy's conversion: every
    fp32 whose low 13 bits (the ones fp16 drops from a normal value) are one
    of the rounding-boundary patterns, over all sign/exponent/high-mantissa
    combinations in fp16's range and beyond it, plus random values and the
    whole subnormal range at a stride."""
    hi = np.arange(0, 1 << 19, dtype=np.uint32) << 13
    lows = np.array([0, 1, 0x0FFF, 0x1000, 0x1001, 0x1FFF], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).reshape(-1)
    # keep |f| below 2^17 (beyond: infinity on both sides, checked separately)
    f = u.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 2.0 ** 17)]
    rng = np.random.default_rng(3)
    f = np.concatenate([f, rng.standard_normal(1 << 20).astype(np.float32) * 1000,
                        (np.arange(1 << 20, dtype=np.float32) * 2.0 ** -34),
                        np.array([65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -25,
                                  np.nextafter(np.float32(2.0 ** -25), np.float32(1))],
                                 np.float32)])
    with np.errstate(over="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    got = orc.convert(f, "fp32", "fp16")
    assert np.array_equal(got, ref), int(np.sum(got != ref))


def _thr_codes(orc, qt, xf, absmax, bs):
    """Independent threshold formulation of the code function on fp32 values:
    numpy IEEE fp32 division, then the rank among round-down fp32 midpoints."""
    cb, codes = _sorted_candidates(orc, qt)
    thr = _rd_thresholds(cb, codes)
    a = np.repeat(absmax, bs)[: xf.size]
    with np.errstate(invalid="ignore", divide="ignore"):
        s = np.where(a == 0, np.float32(0), xf / a).astype(np.float32)
    return np.array(codes)[np.searchsorted(thr, s, side="left")]


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_quantize_fp32_inputs(orc, qt):
    """fp32 inputs (no bf16 rounding): the absmax is numpy's max |x| per block
    and every code agrees with the independent threshold formulation, on
    random blocks and on blocks built to put x / a on both sides of every
    decision midpoint; the exact-rational brute force agrees on a sample."""
    rng = np.random.default_rng(11)
    w = (rng.standard_normal(64 * 400) * 0.02).astype(np.float32)
    cb, codes = _sorted_candidates(orc, qt)
    thr = _rd_thresholds(cb, codes)
    near = []
    for t in thr:  # s = t - 2 ulp .. t + 2 ulp, with a = 1 in element 0
        v = np.float32(t)
        for _ in range(2):
            v = np.nextafter(v, np.float32(-2))
        for _ in range(5):
            near.append(v)
            v = np.nextafter(v, np.float32(2))
    near = np.array(near, np.float32)
    pad = (-(near.size + 1)) % 64
    blk = np.concatenate([[np.float32(1.0)], near, np.zeros(pad, np.float32)]).astype(np.float32)
    w = np.concatenate([w, blk, blk * np.float32(3.0e-5)]).astype(np.float32)
    p, a = orc.quantize_typed(w, "fp32", 64, qt)
    assert np.array_equal(a, np.abs(w).reshape(-1, 64).max(axis=1))
    got = _codes(p, w.size)
    assert np.array_equal(got, _thr_codes(orc, qt, w, a, 64))
    idx = np.random.default_rng(2).integers(0, w.size, 300)
    for i in idx:
        s = np.float32(w[i] / a[i // 64]) if a[i // 64] != 0 else np.float32(0)
        assert got[i] == _brute_nearest(s, cb, codes)


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_quantize_fp16_inputs_every_value(orc, qt):
    """Every finite fp16 value, in blocks whose absmax is fixed by a leading
    element, against the independent threshold formulation."""
    h = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16)
    h = h[np.isfinite(v) & (np.abs(v.astype(np.float32)) <= 1.5)]
    one_half = np.float16(1.5).view(np.uint16)
    rows = h[: h.size - h.size % 63].reshape(-1, 63)
    w = np.concatenate([np.full((rows.shape[0], 1), one_half, np.uint16), rows], axis=1).reshape(-1)
    p, a = orc.quantize_typed(w, "fp16", 64, qt)
    xf = w.view(np.float16).astype(np.float32)
    assert np.all(a == np.float32(1.5))
    assert np.array_equal(_codes(p, w.size), _thr_codes(orc, qt, xf, a, 64))


def test_quantize_typed_bf16_is_the_bf16_path(orc):
    w = workloads.to_u16(workloads.normal_bf16((64 * 50 + 17,), 0.02, 41))
    p1, a1 = orc.quantize(w, 64, "nf4")
    p2, a2 = orc.quantize_typed(w, "bf16", 64, "nf4")
    assert np.array_equal(p1, p2) and np.array_equal(a1, a2)


# ------------------------------------------------ mean-centred double quant


def test_centred_double_quant_worked_examples(orc):
    """Hand-worked, every value exact in fp32 (bs2 = 4):
    a = [254, 0, 190.5, 63.5]: S = (254 + 0) + (190.5 + 63.5) = 508, mu = 127,
      a - mu = [127, -127, 63.5, -63.5], s2 = 127 / 127 = 1, q = [127, -127, 64, -64]
      (half to even), a' = [254, 0, 191, 63];
    a = [254, 0, 190.5, 127]: S = 571.5, mu = 142.875, a - mu = [111.125,
      -142.875, 47.625, -15.875], s2 = 142.875 / 127 = 1.125, q = [99, -127, 42, -14];
    a = [3, 1, 2] (a short last group: padded with a zero for the sum, divided
      by 3): S = (3 + 1) + (2 + 0) = 6, mu = 2, s2 = RN(1/127), q = [127, -127, 0]."""
    q, s2, mu = orc.double_quant_centred(np.array([254, 0, 190.5, 63.5], np.float32), 4)
    assert q.tolist() == [127, -127, 64, -64] and s2.tolist() == [1.0] and mu.tolist() == [127.0]
    q, s2, mu = orc.double_quant_centred(np.array([254, 0, 190.5, 127], np.float32), 4)
    assert q.tolist() == [99, -127, 42, -14] and s2.tolist() == [1.125]
    assert mu.tolist() == [142.875]
    q, s2, mu = orc.double_quant_centred(np.array([3, 1, 2], np.float32), 4)
    assert q.tolist() == [127, -127, 0] and mu.tolist() == [2.0]
    assert s2[0] == f32(1) / f32(127)
    # the dequantized scales a' = RN(RN(q s2) + mu) of the first example
    p = np.array([0xFF, 0xFF], np.uint8)  # code 15 = +1: w = a'
    w32, _ = orc.dequantize(p, 4, 1, "nf4", absmax_q=np.array([127, -127, 64, -64], np.int8),
                            absmax_scale=np.array([1.0], np.float32),
                            absmax_offset=np.array([127.0], np.float32), blocksize2=4)
    assert w32.tolist() == [254.0, 0.0, 191.0, 63.0]


def test_centred_double_quant_invariants(orc):
    """Groups of 256 scales: q in [-127, 127]; the scale farthest from the
    centre maps to +-127; |a' - a| <= s2 / 2 plus the two roundings of a';
    an all-equal group keeps its value exactly (q = 0, a' = mu = a); the
    pairwise sum is within the pairwise-summation bound of the exact sum."""
    from fractions import Fraction as Fr

    rng = np.random.default_rng(8)
    nb = 256 * 4 + 99
    a = (np.abs(rng.standard_normal(nb)) * 0.05).astype(np.float32)
    a[256:512] = np.float32(0.0371)
    q, s2, mu = orc.double_quant_centred(a, 256)
    assert q.dtype == np.int8 and s2.size == mu.size == 5
    for g in range(5):
        blk = a[g * 256:(g + 1) * 256]
        qb = q[g * 256:(g + 1) * 256].astype(np.int64)
        assert np.all((qb >= -127) & (qb <= 127))
        exact = sum(Fr(float(v)) for v in blk)
        bound = 8 * 2.0 ** -24 * float(np.sum(blk)) + 1e-45  # log2(256) levels
        assert abs(float(Fr(float(mu[g])) * len(blk) - exact)) <= bound + len(blk) * float(mu[g]) * 2.0 ** -24
        if g == 1:
            assert mu[g] == np.float32(0.0371) and s2[g] == 0 and np.all(qb == 0)
            continue
        d = np.abs(blk.astype(np.float64) - float(mu[g]))
        assert abs(qb[int(np.argmax(d))]) == 127
        ap = ((qb.astype(np.float32) * s2[g]).astype(np.float32) + mu[g]).astype(np.float32)
        err = np.abs(ap.astype(np.float64) - blk)
        assert np.all(err <= float(s2[g]) / 2 * (1 + 2 ** -14) + 4 * 2.0 ** -24 * float(blk.max()))


# ------------------------------------------------- typed products and dequant


@pytest.mark.parametrize("dtype", ["fp16", "fp32"])
def test_matmul_typed_matches_blas(orc, dtype):
    M, N, K = 3, 29, 160
    rng = np.random.default_rng(5)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    wf = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    if dtype == "fp16":
        x, wc = xf.astype(np.float16).view(np.uint16), wf.astype(np.float16).view(np.uint16)
        xd, wd = x.view(np.float16).astype(np.float64), wc.view(np.float16).astype(np.float64)
    else:
        x, wc, xd, wd = xf, wf, xf.astype(np.float64), wf.astype(np.float64)
    y = orc.matmul_typed(x, wc, dtype)
    ref = xd @ wd.T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("dq", [0, 1, 2])
def test_gemv_typed_equals_dequant_then_matmul(orc, dtype, dq):
    """The direct decode product in each compute dtype equals the oracle's
    dequantize (fp32, or its bf16 / fp16 rounding) followed by its matmul;
    dequantize's fp16 output is numpy's fp16 rounding of the fp32 output."""
    N, K, M = 20, 320, 3
    w = workloads.to_u16(workloads.normal_bf16((N, K), 0.02, 51))
    p, a = orc.quantize(w, 64, "nf4")
    kw = dict(absmax=a)
    if dq == 1:
        q, s2 = orc.double_quant(a, 256)
        kw = dict(absmax_q=q, absmax_scale=s2)
    elif dq == 2:
        q, s2, mu = orc.double_quant_centred(a, 64)
        kw = dict(absmax_q=q, absmax_scale=s2, absmax_offset=mu, blocksize2=64)
    rng = np.random.default_rng(6)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    if dtype == "fp32":
        x = xf
        wc, _ = orc.dequantize(p, N * K, 64, "nf4", **kw)
    else:
        x = orc.convert(xf, "fp32", dtype)
        w32, wc = orc.dequantize(p, N * K, 64, "nf4", half=dtype, **kw)
        if dtype == "fp16":
            assert np.array_equal(wc, w32.astype(np.float16).view(np.uint16))
    y = orc.gemv_quantized_typed(x, p, N, K, 64, "nf4", dtype=dtype, **kw)
    ref = orc.matmul_typed(x, wc.reshape(N, K), dtype)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("dq", [0, 1, 2])
def test_threaded_gemv_is_bitwise_the_sequential_one(orc, dq):
    """The host-thread harness (used only to time the oracle on all cores)
    splits whole rows and runs the sequential code on each share."""
    N, K = 300, 1024
    w = workloads.to_u16(workloads.normal_bf16((N, K), 0.02, 61))
    x = workloads.to_u16(workloads.normal_bf16((3, K), 1.0, 62))
    p, a = orc.quantize(w.reshape(-1), 64, "nf4")
    kw = dict(absmax=a)
    if dq == 1:
        q, s2 = orc.double_quant(a, 256)
        kw = dict(absmax_q=q, absmax_scale=s2)
    elif dq == 2:
        q, s2, mu = orc.double_quant_centred(a, 256)
        kw = dict(absmax_q=q, absmax_scale=s2, absmax_offset=mu)
    y1 = orc.gemv_quantized_typed(x, p, N, K, 64, "nf4", **kw)
    for t in (1, 3, 8):
        assert np.array_equal(orc.gemv_quantized_threads(x, p, N, K, t, 64, "nf4", **kw), y1)
