"""Benchmark of the NF4 hot path on one MI355X.

One step = one pass of the whole path over the 7B-shaped stack (32 layers x
(4 x [4096, 4096] + 3 x [11008, 4096]) bf16 weights, N(0, 0.02^2), NF4 with
double quantization at blocksize 64 by default):
  1. quantize + double-quant every weight (and the prefill weight), one call
     per weight (and, as the separate phase quantize_grouped, the seven weights
     of a layer per call),
  2. dequantize every weight to bf16 (likewise per weight, and per layer as
     dequantize_grouped),
  3. decode GEMV (M = 1, independent seeded x per matrix) through every weight,
     the seven products of a layer in one grouped launch (and, as the separate
     phase gemv_single, one launch per matrix),
  4. the prefill GEMM, X[2048, 4096] . W[14336, 4096]^T (NF4 bs 64 + double
     quant, fp32 accumulation, bf16 output), over --gemm-weights distinct
     seeded weights of that shape back to back (4 by default: a prefill runs
     its layers' GEMMs in a row, so one isolated launch would mostly time the
     clock ramp of an idle GPU),
then the same three stack phases at the other blocksizes of the sweep (128,
256), and the MLP-shaped decode products one matrix per launch: W [11008, 4096]
and [4096, 11008], NF4 bs 64 + double quant, M in {1, 4, 8, 16}, each timed
over a rotation of distinct weights (> 1 GB, so HBM, not the 256 MB last-level
cache, serves them).
Inputs are generated on the GPU from seeded generators and are resident in HBM
before timing. Each phase is captured once in a HIP graph and replayed (or,
with --no-graph, launched eagerly); HIP events between phases give per-phase
device time, which includes the gaps between a phase's launches.

Prints ONE JSON line. `value` is the effective bandwidth of the decode GEMV
phase (algorithmic bytes: 4-bit codes + 8-bit scales + per-group fp32 scales +
x + y, divided by the phase's device time). `roofline` prices the GEMV kernel
against HBM with its average launch duration over the timed region (the phase
time over its launches, so the short gap between two launches is counted in).
The GEMM's TFLOP/s and each phase's own figures are reported next to it,
with roofline fractions against MI355X peaks (HBM 8 TB/s, dense bf16 MFMA
2.5 PFLOP/s). `cpu_baseline` times the CPU oracle's decode GEMV on a bounded
sample of the same workload (test infrastructure, single thread);
`cpu_baselines` does the same for its quantize + double quant, dequantize and
prefill GEMM.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0

# HBM bytes per launch (per call for the prefill: the dequantize launch of the
# weight plus the GEMM) measured by two rocprofv3 counter passes (FETCH_SIZE,
# then WRITE_SIZE, KiB per dispatch) over this benchmark, each scaled by what
# the same counter reads for a plain 1 GiB device copy (FETCH_SIZE x 2.000,
# WRITE_SIZE x 1.000); the summary is profiles/bench_7b_stack_hbm_bytes.md. A
# figure holds only for the kernel sources it was taken on (their SHA-256);
# after any change to one of them the benchmark reports null until the counters
# are taken again.
MEASURED_TRAFFIC = {
    "gemv": ({"gemv1.hip": "765fdc608a7b93162dcbb945341432151cdfb1718232c885eb4acfb046b15a1e"},
             105719270),
    "gemm": ({"dequantize.hip": "1ae016441a333232dba8dbd5b07b9ef38751bc2fd662a64786aec8209bb3e1c9",
              "gemm.hip": "1de4b49fe46fca0f023488a02c9c55bb0985bfae51d97d387f6e373065534135"},
             593958228),
}


def measured_traffic(key):
    import hashlib

    digests, nbytes = MEASURED_TRAFFIC[key]
    for source, digest in digests.items():
        path = os.path.join(ROOT, "bit_weight_quantization_nf4_amd", "csrc", source)
        with open(path, "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != digest:
                return None
    return nbytes


def progress(msg: str) -> None:
    """A progress line on stderr (the JSON result alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--bs", type=int, default=64, choices=[32, 64, 128, 256, 512, 1024, 2048, 4096])
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--gemm-weights", type=int, default=4,
                    help="distinct [14336, 4096] weights the prefill GEMM phase runs through")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample (0 disables it)")
    ap.add_argument("--phases", default="quantize,quantize_grouped,dequantize,dequantize_grouped,"
                                        "gemv,gemv_deps,gemv_single,linear_bias,gemm,gemm_fused,gemm_bias,"
                                        "sweep,mlp,batched,configs",
                    help="comma list of quantize, quantize_grouped, dequantize, dequantize_grouped "
                         "(per matrix / the seven weights of a layer per call), gemv (grouped per "
                         "layer), gemv_deps (grouped as a decoder's dependencies allow: "
                         "{q,k,v}, {o}, {gate,up}, {down} per layer), "
                         "gemv_single (one launch per matrix), linear_bias (the same "
                         "through nf4_linear with a bf16 bias), gemm, gemm_bias (the prefill "
                         "product through nf4_linear with a workspace, without / with a fused "
                         "bias), gemm_fused (the same through nf4_gemm, dequantization fused "
                         "into the GEMM), "
                         "sweep (quantize, dequantize and gemv at the other blocksizes of "
                         "64/128/256), mlp (MLP-shaped decode products at M = 1, 4, 8, 16, 32, "
                         "64), batched (the stack's decode products at M = 4, 16 and 64, a layer "
                         "per grouped launch), configs (the tiny 256x512 workload, the 4096x4096 "
                         "one with 0.1%% outliers x20 and double quant, and the MLP shapes in FP4); "
                         "'copy' adds a plain 1 GiB device copy, the known-size reference "
                         "for HBM byte counters")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch each phase eagerly instead of replaying a captured HIP graph")
    ap.add_argument("--no-split", action="store_true",
                    help="decode products without a workspace: activations that do not fit one "
                         "CU's registers are streamed instead of split along K")
    return ap.parse_args()


def main():
    args = parse()
    split = not args.no_split
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(sharding is described in the design notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_weight_quantization_nf4_amd as nf4
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if nf4.lib().nf4_device_check() != 0:
        raise RuntimeError("device 0 is not gfx950")
    dev = torch.device("cuda", 0)
    bs = args.bs
    requested = args.phases.split(",")
    sweep_bs = [b for b in (64, 128, 256) if b != bs] if "sweep" in requested else []
    mlp_ms = (1, 4, 8, 16, 32, 64) if "mlp" in requested else ()
    batch_ms = (4, 16, 64) if "batched" in requested else ()
    phases = [p for p in requested if p not in ("sweep", "mlp", "batched", "configs")]
    if "configs" in requested:
        phases += ["cfg1_quantize", "cfg1_dequantize", "cfg1_gemv", "cfg2_quantize", "cfg2_gemv"]
        phases += [f"mlp_fp4_{name}_m{m}" for m in (1, 4, 8, 16) for name in ("up", "down")]
    for m in batch_ms:
        phases.append(f"gemv_m{m}")
    for b in sweep_bs:
        phases += [f"quantize_bs{b}", f"dequantize_bs{b}", f"gemv_bs{b}"]
    for m in mlp_ms:
        phases += [f"mlp_up_m{m}", f"mlp_down_m{m}"]

    stack = workloads.stack_7b(args.layers)
    prefill = workloads.PREFILL

    def gpu_normal(shape, sigma, seed):
        g = torch.Generator(device=dev).manual_seed(seed)
        t = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
        if sigma != 1.0:
            t.mul_(sigma)
        return t.to(torch.bfloat16)

    # ---- resident inputs and preallocated outputs
    progress(f"quantizing the {len(stack.matrices)}-matrix stack")
    mats = []
    for m in stack.matrices:
        w = gpu_normal((m.rows, m.cols), m.sigma, m.seed)
        x = gpu_normal((1, m.cols), 1.0, m.seed + 1000)
        qs = nf4.quantize(w, bs, "nf4", double_quant=True)
        # y: the grouped gemv phase's output (the one the oracle re-checks);
        # the per-matrix and bias phases write their own buffers
        mats.append(dict(spec=m, w=w, x=x, qs=qs,
                         wd=torch.empty_like(w),
                         y=torch.empty((1, m.rows), dtype=torch.float32, device=dev),
                         y_single=torch.empty((1, m.rows), dtype=torch.float32, device=dev),
                         y_deps=torch.empty((1, m.rows), dtype=torch.float32, device=dev),
                         y_lin=torch.empty((1, m.rows), dtype=torch.float32, device=dev)))
    # the other blocksizes of the sweep share the bf16 weights and outputs
    for d in mats:
        d["qs_bs"] = {b: nf4.quantize(d["w"], b, "nf4", double_quant=True) for b in sweep_bs}
        d["qs_bs"][bs] = d["qs"]
        d["y_bs"] = {b: torch.empty_like(d["y"]) for b in sweep_bs}
        d["y_bs"][bs] = d["y"]
    pm = prefill.matrices[0]
    pw = gpu_normal((pm.rows, pm.cols), pm.sigma, pm.seed)
    px = gpu_normal((prefill.ms[0], pm.cols), 1.0, prefill.x_seed)
    pqs = nf4.quantize(pw, 64, "nf4", double_quant=True)
    # the GEMM phase's weights: the prefill weight, then seeds pm.seed + 1, ...
    gemm_w = [pqs]
    for r in range(1, args.gemm_weights):
        w = gpu_normal((pm.rows, pm.cols), pm.sigma, pm.seed + r)
        gemm_w.append(nf4.quantize(w, 64, "nf4", double_quant=True))
        del w
    gemm_y = [torch.empty((prefill.ms[0], pm.rows), dtype=torch.bfloat16, device=dev)
              for _ in gemm_w]
    torch.cuda.synchronize()

    # the seven weights of a layer: one grouped launch in the grouped phases
    layers = [mats[i:i + 7] for i in range(0, len(mats), 7)]

    def quantize_at(b, with_prefill):
        def f():
            for d in mats:
                nf4.quantize(d["w"], b, "nf4", True, out=d["qs_bs"][b])
            if with_prefill:
                nf4.quantize(pw, 64, "nf4", True, out=pqs)
        return f

    def quantize_grouped():
        # the same work, the seven weights of a layer in one call
        for grp in layers:
            nf4.quantize_grouped([d["w"] for d in grp], bs, "nf4", True,
                                 outs=[d["qs_bs"][bs] for d in grp])
        nf4.quantize(pw, 64, "nf4", True, out=pqs)

    def dequantize_grouped():
        for grp in layers:
            nf4.dequantize_grouped([d["qs_bs"][bs] for d in grp], outs=[d["wd"] for d in grp])

    def dequantize_at(b):
        def f():
            for d in mats:
                nf4.dequantize(d["qs_bs"][b], out=d["wd"])
        return f


    def gemv_at(b):
        def f():
            for grp in layers:
                nf4.gemv_grouped([d["x"] for d in grp], [d["qs_bs"][b] for d in grp], split=split,
                                 outs=[d["y_bs"][b] for d in grp])
        return f

    # a decoder's layer cannot co-launch its seven products: o waits for the
    # attention of q, k, v and the last MLP product for the first two, so the
    # launches are {q, k, v}, {o}, {gate, up}, {down} (matrices 0-2, 3, 4-5, 6)
    dep_groups = [[0, 1, 2], [3], [4, 5], [6]]

    def gemv_deps():
        for grp in layers:
            for idx in dep_groups:
                sub = [grp[i] for i in idx if i < len(grp)]
                if sub:
                    nf4.gemv_grouped([d["x"] for d in sub], [d["qs"] for d in sub], split=split,
                                     outs=[d["y_deps"] for d in sub])

    def gemv_single():
        # the same products, one launch per matrix (labelled apart from the
        # grouped phase)
        for d in mats:
            nf4.gemv(d["x"], d["qs"], out=d["y_single"], split=split)

    def ph_gemm():
        # nf4_linear with a workspace: at this M the weight is dequantized once
        # into it and the GEMM runs on the dequantized weight
        for q, y in zip(gemm_w, gemm_y):
            nf4.linear(px, q, out=y, split=split)

    def ph_gemm_fused():
        # nf4_gemm: the dequantization fused into the GEMM's weight tiles
        for q, y in zip(gemm_w, gemm_y):
            nf4.gemm(px, q, out=y)

    # the same products through nf4_linear with a bf16 bias per output row
    lin_bias = [gpu_normal((d["spec"].rows,), 0.5, 8000 + i) for i, d in enumerate(mats)]
    gemm_bias = gpu_normal((pm.rows,), 0.5, 8999)

    def linear_bias():
        for d, b in zip(mats, lin_bias):
            nf4.linear(d["x"], d["qs"], b, out_dtype=torch.float32, out=d["y_lin"], split=split)

    def ph_gemm_bias():
        for q, y in zip(gemm_w, gemm_y):
            nf4.linear(px, q, gemm_bias, out=y, split=split)

    # MLP-shaped products, one matrix per launch, rotating over distinct
    # weights: the stack's [11008, 4096] matrices (bs 64), and 48 seeded
    # [4096, 11008] ones
    mlp = {}
    if mlp_ms:
        up = [d["qs_bs"][64] if 64 in d["qs_bs"] else nf4.quantize(d["w"], 64, "nf4", True)
              for d in mats if d["spec"].rows == 11008]
        down = []
        for r in range(48):
            w = gpu_normal((4096, 11008), 0.02, 7000 + r)
            down.append(nf4.quantize(w, 64, "nf4", double_quant=True))
            del w
        for m in mlp_ms:
            for name, qss, N, K in (("up", up, 11008, 4096), ("down", down, 4096, 11008)):
                x = gpu_normal((m, K), 1.0, 7100 + m + K)
                y = torch.empty((m, N), dtype=torch.float32, device=dev)
                mlp[f"mlp_{name}_m{m}"] = dict(qss=qss, x=x, y=y, N=N, K=K, M=m)

    # the other workloads: the tiny [256, 512] weight (NF4 bs 64, no double
    # quant, M = 1; 200 launches back to back on the same cache-resident data:
    # latency-bound), the [4096, 4096] weight with 0.1 % of its entries x20
    # (NF4 bs 64 + double quant, M = 1; 64 distinct seeded copies in rotation,
    # beyond the last-level cache) and the MLP shapes in FP4 (as mlp_*)
    cfg = {}
    if "configs" in requested:
        t = gpu_normal((256, 512), 0.02, 1001)
        cfg["tiny_w"] = t
        cfg["tiny_qs"] = nf4.quantize(t, 64, "nf4", double_quant=False)
        cfg["tiny_x"] = gpu_normal((1, 512), 1.0, 2001)
        cfg["tiny_y"] = torch.empty((1, 256), dtype=torch.float32, device=dev)
        cfg["tiny_wd"] = torch.empty_like(t)
        sq_w, sq_qs = [], []
        for r in range(64):
            g = torch.Generator(device=dev).manual_seed(1002 + 100 * r)
            w = torch.randn((4096, 4096), generator=g, device=dev, dtype=torch.float32).mul_(0.02)
            k = round(0.001 * w.numel())
            go = torch.Generator(device=dev).manual_seed(3002 + 100 * r)
            idx = torch.randperm(w.numel(), generator=go, device=dev)[:k]
            w.view(-1)[idx] *= 20.0
            w = w.to(torch.bfloat16)
            if r < 16:
                sq_w.append(w)  # the quantize phase rotates 16 copies (0.5 GB of bf16)
            sq_qs.append(nf4.quantize(w, 64, "nf4", double_quant=True))
            del w
        cfg["sq_w"], cfg["sq_qs"] = sq_w, sq_qs
        cfg["sq_x"] = gpu_normal((1, 4096), 1.0, 2002)
        cfg["sq_y"] = torch.empty((1, 4096), dtype=torch.float32, device=dev)
        up4 = [nf4.quantize(d["w"], 64, "fp4", True) for d in mats if d["spec"].rows == 11008][:48]
        down4 = []
        for r in range(24):
            w = gpu_normal((4096, 11008), 0.02, 7000 + r)
            down4.append(nf4.quantize(w, 64, "fp4", double_quant=True))
            del w
        for m in (1, 4, 8, 16):
            for name, qss, N, K in (("up", up4, 11008, 4096), ("down", down4, 4096, 11008)):
                x = gpu_normal((m, K), 1.0, 7100 + m + K)
                y = torch.empty((m, N), dtype=torch.float32, device=dev)
                mlp[f"mlp_fp4_{name}_m{m}"] = dict(qss=qss, x=x, y=y, N=N, K=K, M=m)

    def cfg_fn(name):
        def tiny_quantize():
            for _ in range(200):
                nf4.quantize(cfg["tiny_w"], 64, "nf4", False, out=cfg["tiny_qs"])

        def tiny_dequantize():
            for _ in range(200):
                nf4.dequantize(cfg["tiny_qs"], out=cfg["tiny_wd"])

        def tiny_gemv():
            for _ in range(200):
                nf4.gemv(cfg["tiny_x"], cfg["tiny_qs"], out=cfg["tiny_y"], split=split)

        def sq_quantize():
            for w, q in zip(cfg["sq_w"], cfg["sq_qs"]):
                nf4.quantize(w, 64, "nf4", True, out=q)

        def sq_gemv():
            for q in cfg["sq_qs"]:
                nf4.gemv(cfg["sq_x"], q, out=cfg["sq_y"], split=split)
        return dict(cfg1_quantize=tiny_quantize, cfg1_dequantize=tiny_dequantize,
                    cfg1_gemv=tiny_gemv, cfg2_quantize=sq_quantize, cfg2_gemv=sq_gemv)[name]

    # the stack's decode products at batch M, a layer's seven per grouped launch
    # (one activation block per M, shared by the products; an output per product)
    batch = {}
    for m in batch_ms:
        xb = gpu_normal((m, 4096), 1.0, 7300 + m)
        batch[m] = (xb, [torch.empty((m, d["spec"].rows), dtype=torch.float32, device=dev)
                         for d in mats])

    def gemv_batched(m):
        xb, ys = batch[m]

        def f():
            for li, grp in enumerate(layers):
                nf4.gemv_grouped([xb] * len(grp), [d["qs"] for d in grp], split=split,
                                 outs=ys[7 * li:7 * li + len(grp)])
        return f

    def mlp_at(key):
        e = mlp[key]

        def f():
            for q in e["qss"]:
                nf4.gemv(e["x"], q, out=e["y"], split=split)
        return f

    copy_src = copy_dst = None
    if "copy" in phases:
        copy_src = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        copy_dst = torch.empty_like(copy_src)

    def ph_copy():
        copy_dst.copy_(copy_src)

    fns = dict(quantize=quantize_at(bs, True), dequantize=dequantize_at(bs), gemv=gemv_at(bs),
               gemv_single=gemv_single, gemv_deps=gemv_deps, quantize_grouped=quantize_grouped,
               dequantize_grouped=dequantize_grouped,
               gemm=ph_gemm, gemm_fused=ph_gemm_fused, copy=ph_copy, linear_bias=linear_bias,
               gemm_bias=ph_gemm_bias)
    for b in sweep_bs:
        fns[f"quantize_bs{b}"] = quantize_at(b, False)
        fns[f"dequantize_bs{b}"] = dequantize_at(b)
        fns[f"gemv_bs{b}"] = gemv_at(b)
    for key in mlp:
        fns[key] = mlp_at(key)
    for key in ("cfg1_quantize", "cfg1_dequantize", "cfg1_gemv", "cfg2_quantize", "cfg2_gemv"):
        if key in phases:
            fns[key] = cfg_fn(key)
    for m in batch_ms:
        fns[f"gemv_m{m}"] = gemv_batched(m)

    # ---- capture each phase in a graph (after an eager warm-up call)
    progress(f"inputs ready; warm-up call and capture of {len(phases)} phases")
    graphs = {}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for p in phases:
            fns[p]()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for p in phases:
        if args.no_graph:
            graphs[p] = None
            continue
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fns[p]()
        graphs[p] = g
    torch.cuda.synchronize()

    def run(p):
        if graphs[p] is None:
            fns[p]()
        else:
            graphs[p].replay()

    for _ in range(args.warmup):
        for p in phases:
            run(p)
    torch.cuda.synchronize()
    progress(f"captured; timing {args.steps} steps")

    # ---- timed region
    ev = {p: [] for p in phases}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for p in phases:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            run(p)
            b.record()
            ev[p].append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {p: sum(a.elapsed_time(b) for a, b in ev[p]) / args.steps for p in phases}
    ms_sorted = {p: sorted(a.elapsed_time(b) for a, b in ev[p]) for p in phases}


    # ---- algorithmic work per step
    def meta_bytes(n, blocksize):
        nb = -(-n // blocksize)
        return nb + 4 * (-(-nb // 256))  # int8 scale per block + fp32 per 256 blocks

    n_stack = sum(d["spec"].rows * d["spec"].cols for d in mats)
    n_pre = pm.rows * pm.cols
    work = {}

    def quantize_work(b, with_prefill):
        # read bf16, write codes, fp32 absmax, int8 scale and fp32 group scale;
        # blocksizes 64/128/256 do both levels in one pass, the others read
        # the fp32 absmax back in a second launch
        fused = b in (64, 128, 256)
        nbytes, launches = 0, 0
        sizes = [(d["spec"].rows * d["spec"].cols, b) for d in mats]
        if with_prefill:
            sizes.append((n_pre, 64))
        for n, bb in sizes:
            nb = -(-n // bb)
            nbytes += 2 * n + (n + 1) // 2 + 4 * nb + nb + 4 * (-(-nb // 256))
            nbytes += 0 if fused else 4 * nb
            launches += 1 if fused else 2
        return dict(bytes=nbytes, launches=launches)

    def dequantize_work(b):
        return dict(bytes=sum((n + 1) // 2 + meta_bytes(n, b) + 2 * n
                              for n in (d["spec"].rows * d["spec"].cols for d in mats)),
                    launches=len(mats))

    def gemv_work(b):
        nbytes = 0
        for d in mats:
            N, K = d["spec"].rows, d["spec"].cols
            nbytes += N * K // 2 + meta_bytes(N * K, b) + 2 * K + 4 * N
        return dict(bytes=nbytes, launches=len(layers))

    work["quantize"] = quantize_work(bs, True)
    work["dequantize"] = dequantize_work(bs)
    work["quantize_grouped"] = dict(bytes=work["quantize"]["bytes"], launches=len(layers) + 1)
    work["dequantize_grouped"] = dict(bytes=work["dequantize"]["bytes"], launches=len(layers))
    work["gemv"] = gemv_work(bs)
    work["gemv_single"] = dict(bytes=work["gemv"]["bytes"], launches=len(mats))
    work["gemv_deps"] = dict(bytes=work["gemv"]["bytes"],
                             launches=sum(1 for grp in layers for idx in dep_groups
                                          if any(i < len(grp) for i in idx)))
    for b in sweep_bs:
        work[f"quantize_bs{b}"] = quantize_work(b, False)
        work[f"dequantize_bs{b}"] = dequantize_work(b)
        work[f"gemv_bs{b}"] = gemv_work(b)
    for key, e in mlp.items():
        N, K, m = e["N"], e["K"], e["M"]
        per = N * K // 2 + meta_bytes(N * K, 64) + 2 * m * K + 4 * m * N
        work[key] = dict(bytes=per * len(e["qss"]), launches=len(e["qss"]))
    if "configs" in requested:
        n1, n2 = 256 * 512, 4096 * 4096
        nb1 = n1 // 64
        work["cfg1_quantize"] = dict(bytes=200 * (2 * n1 + n1 // 2 + 4 * nb1), launches=200)
        work["cfg1_dequantize"] = dict(bytes=200 * (n1 // 2 + 4 * nb1 + 2 * n1), launches=200)
        work["cfg1_gemv"] = dict(bytes=200 * (n1 // 2 + 4 * nb1 + 2 * 512 + 4 * 256), launches=200)
        nb2 = n2 // 64
        work["cfg2_quantize"] = dict(
            bytes=len(cfg["sq_w"]) * (2 * n2 + n2 // 2 + 4 * nb2 + nb2 + 4 * (-(-nb2 // 256))),
            launches=len(cfg["sq_w"]))
        work["cfg2_gemv"] = dict(
            bytes=len(cfg["sq_qs"]) * (n2 // 2 + meta_bytes(n2, 64) + 2 * 4096 + 4 * 4096),
            launches=len(cfg["sq_qs"]))
    M = prefill.ms[0]
    work["gemm"] = dict(flops=2 * M * pm.rows * pm.cols * len(gemm_w), launches=len(gemm_w))
    work["gemm_bias"] = dict(work["gemm"])
    work["gemm_fused"] = dict(work["gemm"])
    work["linear_bias"] = dict(bytes=work["gemv"]["bytes"] + sum(2 * d["spec"].rows for d in mats),
                               launches=len(mats))
    work["copy"] = dict(bytes=2 * (1 << 30), launches=1)
    for m in batch_ms:
        work[f"gemv_m{m}"] = dict(
            bytes=sum(d["spec"].rows * d["spec"].cols // 2 + meta_bytes(d["spec"].rows * d["spec"].cols, bs)
                      + 2 * m * d["spec"].cols + 4 * m * d["spec"].rows for d in mats),
            launches=len(layers))

    phase_out = {}
    for p in phases:
        t = ms[p] / 1e3
        w = work[p]
        srt = ms_sorted[p]
        spread = dict(ms_median=round(srt[len(srt) // 2], 4), ms_min=round(srt[0], 4))
        if "bytes" in w:
            gbs = w["bytes"] / t / 1e9
            phase_out[p] = dict(ms=round(ms[p], 4), gb_per_s=round(gbs, 1),
                                hbm_frac=round(gbs / HBM_PEAK_GBS, 4), launches=w["launches"],
                                per_launch_us=round(ms[p] * 1e3 / w["launches"], 3),
                                algorithmic_bytes=w["bytes"], **spread)
        else:
            tf = w["flops"] / t / 1e12
            phase_out[p] = dict(ms=round(ms[p], 4), tflops=round(tf, 1),
                                mfma_frac=round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                                launches=w["launches"], flops=w["flops"], **spread)

    gemv_gbs = phase_out.get("gemv", {}).get("gb_per_s")
    result = {
        "metric": "NF4 GEMV effective GB/s (% of HBM peak); NF4 GEMM TFLOP/s (% MFMA peak)",
        "value": gemv_gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0, 0.02^2) bf16 weights, N(0, 1) bf16 activations, on-GPU generators)",
        "config": {
            "workload": f"7B-shaped stack: {args.layers} layers x (4 x [4096,4096] + 3 x "
                        f"[11008,4096]) NF4 bs{bs} + double quant (256); decode GEMV M=1 per "
                        "matrix (the 7 products of a layer in one grouped launch); + prefill GEMM 2048x4096x14336 NF4 bs64 + double quant "
                        f"over {len(gemm_w)} distinct weights back to back",
            "blocksize": bs, "quant_type": "nf4", "double_quant": True, "k_split": split,
            "stack_params": n_stack, "gemv_m": 1, "gemm_mnk": [M, pm.rows, pm.cols],
            "gemm_weights": len(gemm_w),
            "also_timed": "phase gemv_single: the same decode products, one launch per matrix; "
                          "linear_bias / gemm_bias: those products and the prefill GEMM through "
                          "nf4_linear with a fused bf16 bias; gemm_fused: the prefill GEMM "
                          "through nf4_gemm (dequantization fused into the GEMM's weight tiles); "
                          "phases quantize_grouped / dequantize_grouped: the stack's quantize / "
                          "dequantize with the seven weights of a layer in one call; "
                          "phases *_bs128/*_bs256: the stack at the other blocksizes; mlp_*: "
                          "[11008,4096] (up) and [4096,11008] (down) NF4 bs64 + double quant, "
                          "one product per launch over >1 GB of distinct weights, M = 1/4/8/16; "
                          "gemv_m4 / gemv_m16 / gemv_m64: the stack's decode products at M = 4 / "
                          "16 / 64, a layer per grouped launch; gemv_deps: the M = 1 products "
                          "grouped {q,k,v}, {o}, {gate,up}, {down} per layer; cfg1_*: the tiny "
                          "[256,512] workload (latency-bound, 200 launches on cache-resident data); "
                          "cfg2_*: [4096,4096] with 0.1% outliers x20, NF4 bs64 + double quant; "
                          "mlp_fp4_*: the MLP shapes in FP4",
        },
    }
    if "gemv" in phase_out:
        per_launch = work["gemv"]["bytes"] / work["gemv"]["launches"]
        us = ms["gemv"] * 1e3 / work["gemv"]["launches"]
        gbs = per_launch / us / 1e3
        result["roofline"] = {
            "kernel": "gemv1_kernel (NF4 decode GEMV, M=1, one launch per layer of 7 products)",
            "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("gemv"),
            "per_launch_us": round(us, 3),
            "algorithmic_bytes_per_launch": per_launch,
        }
    if "gemm" in phase_out:
        us = ms["gemm"] * 1e3 / work["gemm"]["launches"]
        tf = work["gemm"]["flops"] / work["gemm"]["launches"] / us / 1e6
        result["roofline_gemm"] = {
            "kernel": ("dequantize_kernel + gemm_w16_kernel (NF4 prefill through nf4_linear: the "
                       "weight dequantized once, then the GEMM on it)" if split else
                       "gemm_kernel (NF4 prefill GEMM, dequantization fused)"),
            "bound": "mfma", "achieved": round(tf, 1),
            "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": measured_traffic("gemm") if split else None,
            "per_launch_us": round(us, 3),
        }
    result["phases"] = phase_out

    parity_ok = None
    if args.cpu_seconds > 0:
        result["cpu_baseline"], parity_ok, sample = cpu_baseline(mats, bs, args.cpu_seconds,
                                                                 check="gemv" in phases)
        result["cpu_baseline_all_cores"] = cpu_baseline_threads(sample, bs, args.cpu_seconds / 2)
        result["cpu_baselines"] = cpu_baselines(mats, pw, px, bs, args.cpu_seconds / 2)
    result["parity_ok"] = parity_ok
    print(json.dumps(result), flush=True)
    if parity_ok is False:
        print("bench.py: the GEMV phase's output differs from the oracle beyond the gates",
              file=sys.stderr)
        sys.exit(1)


REL_L2_GATE = 1e-4     # relative L2 error of a product against the fp64 oracle
PER_ELEM_GATE = 1e-3   # per element: |y - y_ref| <= gate * ||w_row|| * ||x||


def cpu_baseline(mats, bs, target_s, check=True):
    """The CPU oracle's decode GEMV on a bounded sample of the same workload: it
    quantizes the sampled weights itself (from the same bf16 inputs), then its
    timed leg is the GEMV, matrix by matrix until ~target_s seconds of work.
    With `check`, its result is also compared, element by element, with the
    output the timed gemv phase left for those matrices (relative L2 <= 1e-4
    and |y - y_ref| <= 1e-3 ||w_row|| ||x|| with w_row the bf16 dequantized
    row). Returns (record, parity_ok or None, the quantized sample for reuse)."""
    import numpy as np

    import oracle
    import workloads

    oracle.ensure_built(force=False)
    done_bytes, done_s, count, worst_rel, worst_elem = 0, 0.0, 0, 0.0, 0.0
    sample = []
    for d in mats:
        N, K = d["spec"].rows, d["spec"].cols
        w16 = workloads.to_u16(d["w"].cpu().reshape(-1))
        x16 = workloads.to_u16(d["x"].cpu())
        p, a = oracle.quantize(w16, bs, "nf4")
        q, s2 = oracle.double_quant(a, 256)
        t = time.perf_counter()
        y = oracle.gemv_quantized(x16, p, N, K, bs, "nf4", absmax_q=q, absmax_scale=s2)
        done_s += time.perf_counter() - t
        sample.append((N, K, x16, p, q, s2))
        nb = -(-(N * K) // bs)
        done_bytes += N * K // 2 + nb + 4 * (-(-nb // 256)) + 2 * K + 4 * N
        if check:
            yg = d["y"].cpu().numpy().astype(np.float64)
            worst_rel = max(worst_rel, float(np.linalg.norm(yg - y) / np.linalg.norm(y)))
            _, wc = oracle.dequantize(p, N * K, bs, "nf4", absmax_q=q, absmax_scale=s2)
            wn = np.linalg.norm((wc.astype(np.uint32) << 16).view(np.float32)
                                .astype(np.float64).reshape(N, K), axis=1)
            xn = np.linalg.norm((x16.astype(np.uint32) << 16).view(np.float32)
                                .astype(np.float64), axis=1)
            ratio = np.abs(yg - y) / (PER_ELEM_GATE * np.outer(xn, wn) + 1e-300)
            worst_elem = max(worst_elem, float(ratio.max()))
        count += 1
        if done_s >= target_s:
            break
    ok = (worst_rel <= REL_L2_GATE and worst_elem <= 1.0) if check else None
    parity = (f"; GPU gemv-phase y vs oracle y: rel-L2 max {worst_rel:.2e} (gate {REL_L2_GATE:g}), "
              f"max |err| / (1e-3 ||w|| ||x||) {worst_elem:.2e} (gate 1)" if check else
              "; gemv phase not run, no parity check")
    model, _, smt = host_info()
    return {
        "value": round(done_bytes / done_s / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": f"oracle decode GEMV (M=1, fp64 sums) over the first {count} matrices of the "
                  f"stack ({done_bytes / 1e6:.1f} MB algorithmic), {done_s:.1f} s single-threaded "
                  f"on {model} (SMT {smt})" + parity,
    }, ok, sample


def host_info():
    """CPU model, logical CPUs this process may use, SMT state (Linux)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    smt = "unknown"
    try:
        with open("/sys/devices/system/cpu/smt/active") as f:
            smt = "on" if f.read().strip() == "1" else "off"
    except OSError:
        pass
    cpus = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return model, cpus, smt


def cpu_baseline_threads(sample, bs, target_s):
    """The same oracle decode GEMV split by rows over every CPU this process
    may use (one host thread each; bitwise the single-threaded result), over
    the matrices the single-threaded leg quantized, in passes until about
    target_s seconds of wall time."""
    import oracle

    model, cpus, smt = host_info()
    done_bytes, done_s, count = 0, 0.0, 0
    while sample and done_s < target_s:
        for N, K, x16, p, q, s2 in sample:
            t = time.perf_counter()
            oracle.gemv_quantized_threads(x16, p, N, K, cpus, bs, "nf4", absmax_q=q,
                                          absmax_scale=s2)
            done_s += time.perf_counter() - t
            nb = -(-(N * K) // bs)
            done_bytes += N * K // 2 + nb + 4 * (-(-nb // 256)) + 2 * K + 4 * N
            count += 1
            if done_s >= target_s:
                break
    return {
        "value": round(done_bytes / max(done_s, 1e-9) / 1e9, 4), "unit": "GB/s", "cores": cpus,
        "kind": "oracle",
        "sample": f"oracle decode GEMV (M=1, fp64 sums) split by rows over {cpus} host threads: "
                  f"{count} products over the single-threaded leg's matrices "
                  f"({done_bytes / 1e6:.1f} MB algorithmic) in {done_s:.1f} s; CPU {model}, "
                  f"SMT {smt}",
    }


def cpu_baselines(mats, pw, px, bs, target_s):
    """The CPU oracle on bounded samples of the other paths, single-threaded, each
    for about target_s seconds: quantize + double quant and dequantize (bf16
    out) over the stack's first matrices, and the prefill GEMM on its first rows
    (the oracle's GEMM is its dequantize of W, timed apart, then an fp64 product
    of those rows)."""
    import oracle
    import workloads

    oracle.ensure_built(force=False)
    out = {}
    q_bytes = q_s = d_bytes = d_s = 0.0
    qcount = dcount = 0
    for d in mats:
        n = d["spec"].rows * d["spec"].cols
        nb = -(-n // bs)
        nb2 = -(-nb // 256)
        w16 = workloads.to_u16(d["w"].cpu().reshape(-1))
        t = time.perf_counter()
        p, a = oracle.quantize(w16, bs, "nf4")
        q, s2 = oracle.double_quant(a, 256)
        q_s += time.perf_counter() - t
        q_bytes += 2 * n + (n + 1) // 2 + 4 * nb + nb + 4 * nb2
        qcount += 1
        if d_s < target_s:
            t = time.perf_counter()
            oracle.dequantize(p, n, bs, "nf4", absmax_q=q, absmax_scale=s2)
            d_s += time.perf_counter() - t
            d_bytes += (n + 1) // 2 + nb + 4 * nb2 + 2 * n
            dcount += 1
        if q_s >= target_s and d_s >= target_s:
            break
    out["quantize"] = {
        "value": round(q_bytes / q_s / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": f"oracle quantize + double quant (NF4 bs {bs}) of the stack's first {qcount} matrices, "
                  f"{q_bytes / 1e6:.0f} MB algorithmic in {q_s:.1f} s"}
    out["dequantize"] = {
        "value": round(d_bytes / d_s / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": f"oracle dequantize to bf16 of the stack's first {dcount} matrices, "
                  f"{d_bytes / 1e6:.0f} MB algorithmic in {d_s:.1f} s"}
    N, K = pw.shape
    w16 = workloads.to_u16(pw.cpu().reshape(-1))
    p, a = oracle.quantize(w16, 64, "nf4")
    q, s2 = oracle.double_quant(a, 256)
    t = time.perf_counter()
    _, wc = oracle.dequantize(p, N * K, 64, "nf4", absmax_q=q, absmax_scale=s2)
    deq_s = time.perf_counter() - t
    wc = wc.reshape(N, K)
    x16 = workloads.to_u16(px.cpu())
    rows, g_s = 0, 0.0
    while g_s < target_s and rows < x16.shape[0]:
        t = time.perf_counter()
        oracle.matmul_bf16(x16[rows:rows + 1], wc)
        g_s += time.perf_counter() - t
        rows += 1
    out["gemm"] = {
        "value": round(2.0 * rows * N * K / g_s / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
        "sample": f"oracle prefill GEMM (fp64 sums): the first {rows} rows of X [{x16.shape[0]}, {K}] times "
                  f"W [{N}, {K}] in {g_s:.1f} s, after its dequantize of W ({deq_s:.1f} s, not counted)"}
    return out


if __name__ == "__main__":
    main()
