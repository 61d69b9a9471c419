"""C-ABI tests that need no GPU: the library loads, exports every symbol the
header declares, its host-side tables match the oracle bit for bit (two
independent derivations), and argument validation rejects bad calls before any
device work. Fake pointers are only ever passed to calls that must fail
validation, or to calls made after the library reported that no device exists.
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nf4.h")

OK, INVALID, UNSUPPORTED, MISALIGNED, DEVICE = 0, 1, 2, 3, 4
A = 0x10000  # a 16-byte-aligned fake address (never dereferenced)
B = 0x20000
MIS = 0x10008


@pytest.fixture(scope="module")
def nf4():
    import bit_weight_quantization_nf4_amd as m

    if not os.path.exists(m.LIB_PATH):
        from bit_weight_quantization_nf4_amd.build import build

        build()
    m.lib()
    return m


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nf4_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(nf4):
    declared = header_functions()
    assert len(declared) == 22
    handle = ctypes.CDLL(nf4.LIB_PATH)
    for name in declared:
        assert hasattr(handle, name), name
    assert sorted(nf4.exported_names()) == declared


def test_version_and_strings(nf4):
    L = nf4.lib()
    assert L.nf4_abi_version() == 3
    for s in range(5):
        assert L.nf4_status_string(s).decode().startswith("NF4_")
    assert b"unknown" in L.nf4_status_string(99)


def test_size_helpers(nf4):
    assert nf4.packed_bytes(0) == 0 and nf4.packed_bytes(7) == 4 and nf4.packed_bytes(8) == 4
    assert nf4.packed_bytes(-1) == -1
    assert nf4.num_blocks(129, 64) == 3 and nf4.num_blocks(0, 64) == 0
    assert nf4.num_blocks(5, 0) == -1


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
def test_library_codebook_equals_oracle(nf4, orc, qt):
    """The library derives its table on the host (Newton on erfc in long
    double / a literal E2M1 list); the oracle by bisection. Same fp32 bits."""
    lib_vals = np.array(nf4.codebook(qt), dtype=np.float32)
    assert np.array_equal(lib_vals.view(np.uint32), orc.codebook(qt).view(np.uint32))


def _desc(nf4, n=4096, bs=64, qt=0, dq=0, bs2=256, packed=A, absmax=B, q=A, s2=B, off=B):
    return nf4.QWeightDesc(packed, absmax, q, s2, n, bs, qt, dq, bs2, off)


def test_quantize_validation(nf4):
    L = nf4.lib()
    q = L.nf4_quantize
    assert q(A, -1, 64, 0, 0, A, B, None, None, None) == INVALID
    assert q(A, 128, 64, 2, 0, A, B, None, None, None) == INVALID
    for bs in (0, 16, 48, 8192):
        assert q(A, 128, bs, 0, 0, A, B, None, None, None) == INVALID
    assert q(None, 128, 64, 0, 0, A, B, None, None, None) == INVALID
    assert q(A, 128, 64, 0, 0, None, B, None, None, None) == INVALID
    assert q(A, 128, 64, 0, 0, A, None, None, None, None) == INVALID
    assert q(A, 128, 64, 0, 1, A, B, None, B, None) == INVALID
    assert q(A, 128, 64, 0, 2, A, B, A, B, None) == INVALID
    assert q(MIS, 128, 64, 0, 0, A, B, None, None, None) == MISALIGNED
    assert q(A, 128, 64, 0, 0, MIS, B, None, None, None) == MISALIGNED
    assert q(A, 128, 64, 0, 1, A, B, MIS, B, None) == MISALIGNED
    assert q(None, 0, 64, 0, 0, None, None, None, None, None) == OK  # empty tensor: no-op


def test_double_quant_validation(nf4):
    dq = nf4.lib().nf4_double_quant
    assert dq(A, -1, 256, A, B, None) == INVALID
    for bs2 in (0, 32, 100, 8192):
        assert dq(A, 10, bs2, A, B, None) == INVALID
    assert dq(None, 10, 256, A, B, None) == INVALID
    assert dq(A, 10, 256, MIS, B, None) == MISALIGNED
    assert dq(None, 0, 256, None, None, None) == OK


def test_dequantize_validation(nf4):
    L = nf4.lib()
    dq = L.nf4_dequantize
    assert dq(None, 0, A, None) == INVALID
    d = _desc(nf4)
    assert dq(ctypes.byref(d), 5, A, None) == INVALID
    assert dq(ctypes.byref(d), 0, None, None) == INVALID
    assert dq(ctypes.byref(d), 0, MIS, None) == MISALIGNED
    for bad in (_desc(nf4, n=-1), _desc(nf4, bs=96), _desc(nf4, qt=3), _desc(nf4, dq=3),
                _desc(nf4, absmax=0), _desc(nf4, dq=1, q=0), _desc(nf4, dq=1, bs2=48),
                _desc(nf4, dq=2, off=0)):
        assert dq(ctypes.byref(bad), 0, A, None) == INVALID
    assert dq(ctypes.byref(_desc(nf4, packed=MIS)), 0, A, None) == MISALIGNED
    assert dq(ctypes.byref(_desc(nf4, dq=1, s2=MIS)), 0, A, None) == MISALIGNED
    assert dq(ctypes.byref(_desc(nf4, dq=2, off=MIS)), 0, A, None) == MISALIGNED
    assert dq(ctypes.byref(_desc(nf4, n=0)), 0, None, None) == OK


@pytest.mark.parametrize("entry", ["nf4_gemv", "nf4_gemm"])
def test_product_validation(nf4, entry):
    fn = getattr(nf4.lib(), entry)
    d = _desc(nf4, n=64 * 128)  # N = 64, K = 128
    call = lambda M, N, K, cd=0, od=1, x=A, y=B, desc=d: fn(x, M, ctypes.byref(desc), N, K, cd, od, y, None)  # noqa: E731
    assert call(1, 64, 100) == INVALID  # N*K != n
    assert call(-1, 64, 128) == INVALID
    assert call(1, 64, 128, od=4) == INVALID
    assert call(1, 64, 128, cd=9) == INVALID
    assert call(1, 64, 128, cd=3) == INVALID
    assert call(1, 64, 128, x=None) == INVALID
    assert call(1, 64, 128, y=MIS) == MISALIGNED
    d96 = _desc(nf4, n=64 * 96, bs=64)
    assert call(1, 64, 96, desc=d96) == UNSUPPORTED  # K % blocksize != 0
    assert call(0, 64, 128, x=None, y=None) == OK
    if entry == "nf4_gemv":
        assert call(65, 64, 128) == INVALID  # past the decode range


def test_grouped_validation(nf4):
    L = nf4.lib()
    P = ctypes.c_void_p
    d = (nf4.QWeightDesc * 2)(_desc(nf4, n=64 * 128), _desc(nf4, n=64 * 256))
    xs = (P * 2)(A, A)
    ys = (P * 2)(B, B)
    Ns = (ctypes.c_int32 * 2)(64, 64)
    Ks = (ctypes.c_int32 * 2)(128, 256)
    g = L.nf4_gemv_grouped
    assert g(17, xs, 1, d, Ns, Ks, 0, 1, ys, None) == INVALID
    assert g(-1, xs, 1, d, Ns, Ks, 0, 1, ys, None) == INVALID
    assert g(2, None, 1, d, Ns, Ks, 0, 1, ys, None) == INVALID
    assert g(2, xs, 65, d, Ns, Ks, 0, 1, ys, None) == INVALID
    assert g(0, None, 1, None, None, None, 0, 1, None, None) == OK
    Kbad = (ctypes.c_int32 * 2)(128, 100)
    assert g(2, xs, 1, d, Ns, Kbad, 0, 1, ys, None) == INVALID  # second product N*K != n
    mixed = (nf4.QWeightDesc * 2)(_desc(nf4, n=64 * 128), _desc(nf4, n=64 * 256, qt=1))
    assert g(2, xs, 1, mixed, Ns, Ks, 0, 1, ys, None) == UNSUPPORTED
    ys_bad = (P * 2)(B, MIS)
    assert g(2, xs, 1, d, Ns, Ks, 0, 1, ys_bad, None) == MISALIGNED


def test_quantize_ex_validation(nf4):
    q = nf4.lib().nf4_quantize_ex
    #        w, dtype, rows, cols, ld, bs, qt, dq, packed, absmax, q, s2, off, stream
    ok = dict(w=A, dt=0, rows=4, cols=64, ld=64, bs=64, qt=0, dq=0, p=A, a=B, qq=None, s2=None,
              off=None)

    def call(**kw):
        a = {**ok, **kw}
        return q(a["w"], a["dt"], a["rows"], a["cols"], a["ld"], a["bs"], a["qt"], a["dq"],
                 a["p"], a["a"], a["qq"], a["s2"], a["off"], None)

    assert call(dt=3) == INVALID
    assert call(rows=-1) == INVALID
    assert call(ld=32) == INVALID                      # ld < cols
    assert call(dq=3) == INVALID
    assert call(dq=2, qq=A, s2=B) == INVALID           # centred mode needs the offsets
    assert call(dq=1) == INVALID                       # no absmax_q / absmax_scale
    assert call(cols=60, ld=64) == UNSUPPORTED         # a strided row of 60 elements
    assert call(ld=68) == MISALIGNED                   # rows 136 bytes apart
    assert call(w=MIS) == MISALIGNED
    assert call(dq=2, qq=A, s2=B, off=MIS) == MISALIGNED
    assert call(w=None, rows=0) == OK                  # empty matrix: no-op


def test_double_quant_ex_validation(nf4):
    dq = nf4.lib().nf4_double_quant_ex
    assert dq(A, 10, 256, 0, A, B, A, None) == INVALID      # mode none
    assert dq(A, 10, 256, 3, A, B, A, None) == INVALID
    assert dq(A, 10, 256, 2, A, B, None, None) == INVALID   # centred without offsets
    assert dq(A, 10, 256, 2, A, B, MIS, None) == MISALIGNED
    assert dq(None, 0, 256, 2, None, None, None, None) == OK


def test_linear_ex_validation(nf4):
    fn = nf4.lib().nf4_linear_ex
    d = _desc(nf4, n=64 * 128)  # N = 64, K = 128
    call = lambda M, ldx, ldy, cd=0, bias=None: fn(A, ldx, M, ctypes.byref(d), 64, 128, bias, cd, 1, B, ldy, None)  # noqa: E731
    assert call(2, 100, 64) == INVALID        # ldx < K
    assert call(2, 128, 32) == INVALID        # ldy < N
    assert call(2, 132, 64) == MISALIGNED     # x rows 264 bytes apart
    assert call(2, 128, 64, bias=A + 1) == MISALIGNED
    assert call(2, 128, 64, cd=2, bias=A + 1) == MISALIGNED
    assert call(2, 1 << 30, 64) == UNSUPPORTED  # x beyond 31-bit offsets


def test_no_device_is_reported(nf4):
    """With no HIP device, a valid call reports NF4_ERR_DEVICE (checked only
    when the library itself says no device is present)."""
    L = nf4.lib()
    if L.nf4_device_check() != DEVICE:
        pytest.skip("a HIP device is present")
    assert L.nf4_quantize(A, 128, 64, 0, 0, A, B, None, None, None) == DEVICE
    d = _desc(nf4, n=64 * 128)
    assert L.nf4_gemv(A, 1, ctypes.byref(d), 64, 128, 0, 1, B, None) == DEVICE


def test_oracle_build_callable_after_submodule_import():
    # importing the build submodule must not shadow the package's build call
    # (build() and smoke() may run in one process)
    import oracle
    import oracle.build  # noqa: F401

    assert oracle.ensure_built(force=False).endswith("libnf4_oracle.so")
    assert oracle.ensure_built(force=False).endswith("libnf4_oracle.so")


def test_workspace_bytes_query(nf4):
    """nf4_linear_workspace_bytes: zero where the dispatch uses none (the
    single-row kernel, x that fits one CU's registers, fp32 compute, the GEMM
    below 1536 rows, more K ranges than the kernel takes); S * M * N * 4
    rounded up to 256 for a decode K split (S K ranges of at most 48 / 32 / 16
    chunks of 128 codes at M <= 16 / 32 / 64; up to M = 8 the register-
    resident kernel streams x instead; from 8 rows, a product whose x would
    take two or more such ranges (three or more from 17 rows) takes the tiled
    kernel's split instead);
    2 * N * K rounded up to 256 for a prefill product of 1536 rows or more (the
    weight dequantized once)."""
    q = nf4.lib().nf4_linear_workspace_bytes
    BF, F32, F16 = 0, 1, 2
    assert q(1, 4096, 11008, 64, BF, F32, 1) == 0          # single-row kernel
    assert q(16, 4096, 6144, 64, BF, F32, 1) == 0          # 48 chunks fit
    # 9..16 rows with x past one CU: the tiled kernel's split (ranges of at
    # most 16 chunks, as many as keep one round of workgroups, two per CU, on
    # 256 CUs)
    assert q(16, 4096, 6272, 64, BF, F32, 1) == 7 * 16 * 4096 * 4  # 49 chunks -> 7 x 7
    assert q(16, 4096, 11008, 64, BF, BF, 1) == 8 * 16 * 4096 * 4
    assert q(1, 4096, 11008, 64, F16, F16, 1) == 0         # M <= 8 streams x
    # 8 rows with x past two ranges of the register-resident kernel: the tiled
    # kernel (64-row blocks, two workgroups per CU: 64 blocks x 8 ranges)
    assert q(8, 4096, 11008, 64, BF, F32, 1) == 8 * 8 * 4096 * 4
    assert q(7, 4096, 11008, 64, BF, F32, 1) == 0          # M <= 7 streams x
    assert q(8, 4096, 6144, 64, BF, F32, 1) == 0           # 48 chunks fit
    assert q(9, 100, 11008, 64, BF, BF, 2) == (8 * 9 * 100 * 4 + 255) // 256 * 256  # centred
    assert q(32, 11008, 4096, 64, BF, F32, 1) == 0
    assert q(32, 11008, 4224, 64, BF, F32, 1) == 2 * 32 * 11008 * 4
    assert q(64, 11008, 4096, 64, BF, F32, 1) == 2 * 64 * 11008 * 4
    # three or more ranges at 17..64 rows: the tiled kernel's split, ranges of
    # at most 16 chunks, as many as keep one round of workgroups on 256 CUs
    # (32 blocks of 128 rows -> 8) and the partial sums within the codes' size
    assert q(64, 4096, 11008, 64, BF, F32, 1) == 8 * 64 * 4096 * 4
    assert q(32, 4096, 11008, 64, BF, BF, 1) == 8 * 32 * 4096 * 4
    assert q(64, 21846, 11008, 64, BF, F32, 1) == 6 * 64 * 21846 * 4  # 171 blocks: 86 / 16 -> 6
    assert q(64, 4096, 5120, 64, BF, F32, 1) == 5 * 64 * 4096 * 4     # cap K / (16 M) = 5
    assert q(40, 33, 2176, 64, BF, F32, 0) == (2 * 40 * 33 * 4 + 255) // 256 * 256
    assert q(64, 4096, 2048, 64, BF, F32, 1) == 0
    assert q(64, 4096, 1 << 20, 64, BF, F32, 1) == 0      # beyond 8 K ranges: x streams
    assert q(65, 4096, 11008, 64, BF, F32, 1) == 0         # the GEMM, dequantizing per tile
    assert q(1535, 14336, 4096, 64, BF, BF, 1) == 0
    # from 1536 rows: the weight dequantized once (2 N K bytes, rounded up to 256)
    assert q(1536, 14336, 4096, 64, BF, BF, 1) == 2 * 14336 * 4096
    assert q(2048, 100, 96, 32, F16, F32, 2) == (2 * 100 * 96 + 255) // 256 * 256
    assert q(2048, 14336, 4096, 64, F32, F32, 1) == 0      # fp32 compute
    assert q(16, 4096, 11008, 64, F32, F32, 1) == 0        # fp32 compute
    assert q(0, 4096, 11008, 64, BF, F32, 1) == 0


def test_workspace_argument_validation(nf4):
    L = nf4.lib()
    d = _desc(nf4, n=64 * 128)  # N = 64, K = 128
    lin = lambda M, ws, nb: L.nf4_linear_ws(A, 128, M, ctypes.byref(d), 64, 128, None, 0, 1, B, 64, ws, nb, None)  # noqa: E731
    assert lin(2, None, -1) == INVALID
    assert lin(2, None, 256) == INVALID       # bytes without a workspace
    assert lin(2, MIS, 256) == MISALIGNED
    assert lin(100, None, 256) == INVALID     # the GEMM path checks it too
    assert lin(0, None, 0) == OK              # M = 0: no-op
    X = (ctypes.c_void_p * 1)(A)
    Y = (ctypes.c_void_p * 1)(B)
    Ns = (ctypes.c_int32 * 1)(64)
    Ks = (ctypes.c_int32 * 1)(128)
    g = lambda ws, nb: L.nf4_gemv_grouped_ws(1, X, 0, ctypes.byref(d), Ns, Ks, 0, 1, Y, ws, nb, None)  # noqa: E731
    assert g(None, -5) == INVALID
    assert g(MIS, 16) == MISALIGNED
    assert g(None, 0) == OK
