"""NF4_LOG=1: the library writes one "[nf4] ..." line per dispatch decision to
stderr (the kernel a call takes, with its shape and workspace); without the
variable it writes nothing. Run in a child process, since the variable is
read once per process."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import torch
import bit_weight_quantization_nf4_amd as nf4
g = torch.Generator(device="cuda").manual_seed(1)
w = (torch.randn(448, 11008, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
qs = nf4.quantize(w, 64, "nf4", double_quant=True)
nf4.dequantize(qs, torch.bfloat16)
for M in (1, 4, 16, 32):
    x = torch.randn(M, 11008, device="cuda", generator=g).to(torch.bfloat16)
    nf4.linear(x, qs, out_dtype=torch.float32)
x = torch.randn(1536, 11008, device="cuda", generator=g).to(torch.bfloat16)
nf4.linear(x, qs)
nf4.linear(x, qs, split=False)
torch.cuda.synchronize()
print("child done", flush=True)
"""


def _run(env_extra):
    env = dict(os.environ)
    env.pop("NF4_LOG", None)
    env.update(env_extra)
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    return subprocess.run([sys.executable, "-c", SCRIPT], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=240)


def test_log_lines_name_each_dispatch():
    r = _run({"NF4_LOG": "1"})
    assert r.returncode == 0, r.stderr[-2000:]
    assert "child done" in r.stdout
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("[nf4] ")]
    text = "\n".join(lines)
    assert "quantize 1 tensor(s) (first n=4931584) bs=64: quantize_dq_kernel" in text, text
    assert "dequantize 1 tensor(s) (first n=4931584) out_dtype=0: dequantize_kernel" in text, text
    assert "decode M=1: gemv1_kernel" in text, text
    assert "decode M=4 K=11008: gemv_mt_kernel (x streamed)" in text, text
    # 448 rows = 7 blocks of 64 at M = 16 (two workgroups per CU): 8 K ranges
    assert ("decode M=16 K=11008: gemv_tk_kernel (x staged in LDS; first product in 8 K range(s) "
            "of 11 chunks), 6 steps, grid 56 x 1, then gemv_split_reduce_kernel") in text, text
    # 448 rows = 4 blocks of 128: 8 K ranges (at most K / (16 M) = 21), 11 chunks each
    assert ("decode M=32 K=11008: gemv_tk_kernel (x staged in LDS; first product in 8 K range(s) "
            "of 11 chunks), 6 steps, grid 32 x 1, then gemv_split_reduce_kernel") in text, text
    assert "prefill M=1536 N=448 K=11008 bs=64: dequantize once into the workspace" in text, text
    assert "prefill M=1536 N=448 K=11008 bs=64: gemm_kernel (dequantization fused)" in text, text


def test_tiled_decode_switch():
    """NF4_DECODE_TILED=0 keeps 16- and 32-row products on the register-
    resident kernel's split (2 / 3 K ranges of at most 48 / 32 chunks)."""
    r = _run({"NF4_LOG": "1", "NF4_DECODE_TILED": "0"})
    assert r.returncode == 0, r.stderr[-2000:]
    text = "\n".join(ln for ln in r.stderr.splitlines() if ln.startswith("[nf4] "))
    assert "gemv_tk_kernel" not in text, text
    assert "decode M=32 K=11008: gemv_mtx_kernel with 2 row tile(s), K split into 3 ranges" in text, \
        text
    assert "decode M=16 K=11008: gemv_mtx_kernel with 1 row tile(s), K split into 2 ranges" in text, \
        text


def test_no_log_without_the_variable():
    r = _run({})
    assert r.returncode == 0, r.stderr[-2000:]
    assert "[nf4]" not in r.stderr
