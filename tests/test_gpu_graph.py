"""The C-ABI calls under HIP graph capture: quantize with double quant,
dequantize, a grouped M = 1 decode call, the K-split decode products (their
workspace allocated by torch during capture), the prefill GEMM and a 1536-row
prefill product that dequantizes its weight into a workspace, captured
once and replayed several times with eager work and synchronisations between
the replays; every replay must equal the eager results bit for bit."""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nf4():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_weight_quantization_nf4_amd as m

    assert m.lib().nf4_device_check() == 0, "device is not gfx950"
    return m


def _run(nf4, w_up, w_down, xs):
    """Every call once; returns the outputs (new tensors)."""
    qu = nf4.quantize(w_up, 64, "nf4", double_quant=True)
    qd = nf4.quantize(w_down, 64, "nf4", double_quant=True)
    out = [qu.packed, qu.absmax_q, qu.absmax_scale, qd.packed]
    out.append(nf4.dequantize(qd, torch.bfloat16))
    out += nf4.gemv_grouped([xs["m1_up"], xs["m1_down"]], [qu, qd], torch.float32)
    out.append(nf4.linear(xs["m16_down"], qd, xs["bias_down"], out_dtype=torch.float32))  # tiled, 8 ranges
    out.append(nf4.linear(xs["m64_up"], qu, None, out_dtype=torch.bfloat16))              # 2 K ranges
    out.append(nf4.linear(xs["m40_down"], qd, None, out_dtype=torch.float32))             # tiled, 8 ranges
    out.append(nf4.gemm(xs["prefill"], qu, torch.bfloat16))
    # 1536 rows with a workspace: the weight dequantized once, then the GEMM
    out.append(nf4.linear(xs["prefill_long"], qd, out_dtype=torch.bfloat16))
    return out


def test_graph_replays_equal_eager(nf4):
    w_up = workloads.normal_bf16((11008, 4096), 0.02, 4401).cuda()
    w_down = workloads.normal_bf16((4096, 11008), 0.02, 4402).cuda()
    xs = {
        "m1_up": workloads.normal_bf16((1, 4096), 1.0, 4403).cuda(),
        "m1_down": workloads.normal_bf16((1, 11008), 1.0, 4404).cuda(),
        "m16_down": workloads.normal_bf16((16, 11008), 1.0, 4405).cuda(),
        "bias_down": workloads.normal_bf16((4096,), 0.5, 4406).cuda(),
        "m64_up": workloads.normal_bf16((64, 4096), 1.0, 4407).cuda(),
        "m40_down": workloads.normal_bf16((40, 11008), 1.0, 4408).cuda(),
        "prefill": workloads.normal_bf16((300, 4096), 1.0, 4409).cuda(),
        "prefill_long": workloads.normal_bf16((1536, 11008), 1.0, 4410).cuda(),
    }
    eager = _run(nf4, w_up, w_down, xs)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _run(nf4, w_up, w_down, xs)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = _run(nf4, w_up, w_down, xs)
    for rep in range(3):
        for t in captured:
            t.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(captured, eager)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (rep, k)
        # eager work between replays
        again = _run(nf4, w_up, w_down, xs)
        torch.cuda.synchronize()
        for a, b in zip(again, eager):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
