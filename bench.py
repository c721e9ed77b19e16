"""Throughput of the NF4 / QLoRA-linear hot path on one MI355X.

One step = one pass of the whole path over one batch of the single
4096x4096 projection workload (W ~ N(0, 0.02) in fp32, LoRA r = 16,
alpha = 32):

  quantise W (fp32 -> NF4 codes + fp32 absmax)      nf4_quantize
  double-quantise the absmax                         nf4_double_quant
  dequantise a weight to bf16                        nf4_dequant
  decode forward, X: 1 x 4096                        qlora_linear_fwd (M = 1)
  prefill forward, X: 2048 x 4096                    qlora_linear_fwd (M = 2048)
  backward at M = 2048 (dX, dA, dB)                  qlora_linear_bwd

Inputs are synthetic, generated on the device before the timed region.  Four
weight slots rotate: step i quantises slot i % 4 while the forward/backward
read slot (i + 2) % 4, quantised two steps earlier, so weight reads come from
HBM rather than from a cache that still holds what the quantiser just wrote.

The step is captured once per slot phase into a HIP graph (the library only
enqueues kernels on the current stream, so capture records them), and the
timed region replays the graphs: the ~15 launches of a step then run without
host launch gaps.  `value` is the step's algorithmic contraction work
(prefill forward + backward + decode GEMV, FLOPs counted as 2 per
multiply-add, dequant work not counted) divided by the step time.

Each stage is then timed alone (`stages.stage_us_graph`): a graph of
back-to-back calls of that stage, replayed between two HIP events; the
bandwidth-bound stages cycle through more distinct buffers than the
Infinity Cache holds.  The quantise and decode figures of `metrics` come from
these loops (per call, so the decode figure includes its epilogue kernel).

A second, eager pass over the same steps enables the library's kernel trace:
HIP events recorded around each call's dominant kernel on its own launch
stream.  Its per-kernel average durations give the per-stage figures in
`stages` and the `roofline` object (for the kernel with the largest share of
the step).  `cpu_baseline` times the CPU oracle on a bounded sample.

`roofline.traffic` is the HBM bytes per launch of that kernel read from
rocprofv3 FETCH_SIZE and WRITE_SIZE counters (table `TRAFFIC` below, each
counter scaled by what it reads for a plain copy of known size, taken with
`--copy-calibration`); it is null when no such measurement exists for the
kernel source as it is now.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
N, K, R, ALPHA = 4096, 4096, 16, 32.0
M_DEC, M_PRE = 1, 2048
SLOTS = 4
STAGE_REPS, STAGE_REPLAYS = 8, 5
CSRC = os.path.join(ROOT, "bit_nf4_quantized_08_amd", "csrc")
KERNEL_SOURCE = {
    "quantize": "k_codec.hip", "double_quant": "k_codec.hip", "dequant": "k_codec.hip",
    "gemv": "k_linear.hip", "gemm_fwd": "k_qgemm.hip", "gemm_dx": "k_qgemm.hip",
    "lowrank": "k_lowrank.hip", "gemm_db": "k_lowrank.hip", "gemm_da": "k_lowrank.hip",
}
# Measured HBM bytes per launch: rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per
# dispatch), each scaled by the ratio of known bytes to counted bytes for a 256 MiB
# copy in the same run.  Keyed by kernel; `sha256` is that of the kernel's source
# file and qn_device.h when the counters were taken.
TRAFFIC = {  # profiles/qlora_step_4096_hbm_traffic.md
    "dequant": {"bytes": 42277971, "sha256": "64942f24ec708f7693c38b703cf180ff08c4ebac7e360d443a7c99e630a68bd8"},
    "double_quant": {"bytes": 1372125, "sha256": "64942f24ec708f7693c38b703cf180ff08c4ebac7e360d443a7c99e630a68bd8"},
    "gemv": {"bytes": 9061826, "sha256": "3dd0a326c81211bd432891d82b61327f1b245ee240598c45690d9ef94acefed1"},
    "gemm_fwd": {"bytes": 85964666, "sha256": "a2a3370f8763a396d8a12159f88d6692a8a160dde4b3237fa6fc8f8e4ef0410b"},
    "gemm_dx": {"bytes": 87147262, "sha256": "a2a3370f8763a396d8a12159f88d6692a8a160dde4b3237fa6fc8f8e4ef0410b"},
    "quantize": {"bytes": 76629421, "sha256": "64942f24ec708f7693c38b703cf180ff08c4ebac7e360d443a7c99e630a68bd8"},
    "lowrank": {"bytes": 27061116, "sha256": "0587280805dc337581ae803574baa2f2398fc9fae7da96d91f1c6910fbda4453"},
    "gemm_db": {"bytes": 43088798, "sha256": "0587280805dc337581ae803574baa2f2398fc9fae7da96d91f1c6910fbda4453"},
}


def source_sha(kind):
    h = hashlib.sha256()
    for f in (KERNEL_SOURCE[kind], "qn_device.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic(kind):
    t = TRAFFIC.get(kind)
    if t is None or t["sha256"] != source_sha(kind):
        return None
    return t["bytes"]


# Linear projections (N, K) of one transformer layer of each model shape.
QWEN_LINEARS = {"q": (3584, 3584), "k": (512, 3584), "v": (512, 3584), "o": (3584, 3584),
                "gate": (18944, 3584), "up": (18944, 3584), "down": (3584, 18944)}
L70B_LINEARS = {"q": (8192, 8192), "k": (1024, 8192), "v": (1024, 8192), "o": (8192, 8192),
                "gate": (28672, 8192), "up": (28672, 8192), "down": (8192, 28672)}


def layer_times(lib, dev, stream, linears, r, M, bwd):
    """Forward (and backward) time of all linears of one layer at M tokens:
    seeded N(0, 0.02) weights in NF4 with double quantisation, one graph of the
    layer's calls, replayed; TFLOP/s over the layer's algorithmic FLOPs."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(4096 + r)
    rnd = lambda shape, std: (torch.randn(shape, generator=g, device=dev) * std).to(torch.bfloat16)
    items = []
    for name, (N, K) in linears.items():
        w = lib.quantize_weight(rnd((N, K), 0.02))
        X, A, B = rnd((M, K), 1.0), rnd((r, K), 0.01), rnd((N, r), 0.01)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        it = dict(N=N, K=K, w=w, X=X, A=A, B=B, Y=Y, wsf=lib.workspace(lib.QN_OP_FWD, M, N, K, r, dev))
        if bwd:
            it.update(dY=rnd((M, N), 1.0), dX=torch.empty((M, K), dtype=torch.bfloat16, device=dev),
                      dA=torch.empty((r, K), dtype=torch.bfloat16, device=dev),
                      dB=torch.empty((N, r), dtype=torch.bfloat16, device=dev),
                      wsb=lib.workspace(lib.QN_OP_BWD, M, N, K, r, dev))
        items.append(it)
    alpha = 2.0 * r

    def run(kind):
        for it in items:
            if kind == "fwd":
                lib.qlora_linear_fwd(it["X"], it["w"], it["A"], it["B"], alpha, Y=it["Y"], ws=it["wsf"])
            else:
                lib.qlora_linear_bwd(it["dY"], it["X"], it["w"], it["A"], it["B"], alpha,
                                     out=(it["dX"], it["dA"], it["dB"]), ws=it["wsb"])

    out = {}
    for kind in (("fwd", "bwd") if bwd else ("fwd",)):
        run(kind)
        torch.cuda.synchronize()
        sg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(sg, stream=stream):
            run(kind)
        sg.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(3):
                sg.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 3
        if kind == "fwd":
            flops = sum(2 * M * it["N"] * it["K"] + 2 * M * r * (it["K"] + it["N"]) for it in items)
        else:
            flops = sum(2 * M * it["N"] * it["K"] + 4 * M * r * (it["K"] + it["N"]) for it in items)
        out[kind + "_us"] = round(us, 1)
        out[kind + "_TFLOPs"] = round(flops / (us * 1e-6) / 1e12, 1)
        del sg
    del items
    return out


def sizes():
    n = N * K
    nb = n // 64
    ng = (nb + 255) // 256
    w_bytes = n // 2 + nb + 4 * ng
    return dict(
        n=n, nb=nb, ng=ng,
        quantize_bytes=4 * n + n // 2 + 4 * nb,
        dq_bytes=4 * nb + nb + 4 * ng,
        dequant_bytes=w_bytes + 2 * n,
        gemv_weight_bytes=w_bytes,
        gemv_all_bytes=w_bytes + 2 * K * M_DEC + 2 * N * M_DEC + 2 * R * K + 2 * N * R,
        gemv_flops=2 * M_DEC * N * K + 2 * M_DEC * K * R + 2 * M_DEC * R * N,
        fwd_flops=2 * M_PRE * N * K + 2 * M_PRE * K * R + 2 * M_PRE * R * N,
        fwd_gemm_kernel_flops=2 * M_PRE * N * K + 2 * M_PRE * R * N,
        bwd_flops=2 * M_PRE * N * K + 4 * M_PRE * N * R + 4 * M_PRE * R * K,
        dx_gemm_kernel_flops=2 * M_PRE * N * K + 2 * M_PRE * R * K,
        # low-rank products: one launch in the forward (H = X A^T -> s H bf16), one
        # in the backward (dH = s dY B -> dH and dH^T; H -> (s H)^T); operands read
        # once, outputs written once.  The trace averages the two launches.
        lowrank_fwd_bytes=2 * M_PRE * K + 2 * R * K + 2 * M_PRE * R,
        lowrank_bwd_bytes=(2 * M_PRE * N + 2 * R * N + 4 * M_PRE * R) + (2 * M_PRE * K + 2 * R * K + 2 * M_PRE * R),
        # column reductions dA = dH^T X and dB = (s H)^T dY in one launch: X, dY
        # and the two transposed factors read once (its per-split partial sums are
        # an implementation choice, not counted)
        colred_bytes=2 * M_PRE * (K + N) + 4 * R * M_PRE,
    )


def cpu_baseline(min_seconds=12.0, max_steps=24):
    """Time the CPU oracle on a bounded sample of the same workload: whole oracle
    steps (quantise, double quant and bf16 dequant of one 4096x4096 fp32 weight,
    then the step's fp64 contractions: decode M=1, prefill M=2048 forward and
    backward) repeated until `min_seconds` have passed.  The value is the step's
    contraction FLOPs over the oracle's step time, as for the GPU figure."""
    import numpy as np
    import oracle
    from bit_nf4_quantized_08_amd import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    s = sizes()
    X = synth.bf16_values(synth.to_bf16(synth.gaussian((M_PRE, K), 1.0, synth.SEED_X)))
    A = synth.bf16_values(synth.to_bf16(synth.gaussian((R, K), 0.01, synth.SEED_A)))
    B = synth.bf16_values(synth.to_bf16(synth.gaussian((N, R), 0.01, synth.SEED_B)))
    dY = synth.bf16_values(synth.to_bf16(synth.gaussian((M_PRE, N), 1.0, synth.SEED_DY)))
    t_codec = t_q = t_mm = 0.0
    steps = 0
    while steps < max_steps and (steps < 2 or t_codec + t_mm < min_seconds):
        W = synth.gaussian((N, K), 0.02, synth.SEED_BULK0 + steps)
        t0 = time.perf_counter()
        packed, absmax, _ = oracle.quantize(W)
        t1 = time.perf_counter()
        k, step = oracle.double_quant(absmax)
        Wh = oracle.dequant_bf16_weight(packed, N, K, oracle.dq_absmax(k, step))
        t2 = time.perf_counter()
        oracle.forward(X[:M_DEC], Wh, A, B, ALPHA)
        oracle.forward(X, Wh, A, B, ALPHA)
        oracle.backward(dY, X, Wh, A, B, ALPHA)
        t3 = time.perf_counter()
        t_q += t1 - t0
        t_codec += t2 - t0
        t_mm += t3 - t2
        steps += 1
    flops = s["gemv_flops"] + s["fwd_flops"] + s["bwd_flops"]
    return {
        "value": flops * steps / (t_codec + t_mm) / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": (f"{steps} whole oracle steps of the same workload in {t_codec + t_mm:.1f} s: codec "
                   f"(quantise, double quant, bf16 dequant of a fresh 4096x4096 fp32 weight) "
                   f"{t_codec / steps:.2f} s/step on 1 core, fp64 contractions {t_mm / steps:.2f} s/step "
                   f"on {blas_threads} BLAS threads"),
        "ms_per_step": (t_codec + t_mm) * 1e3 / steps,
        "quantize_GBps": steps * s["quantize_bytes"] / t_q / 1e9,
        "host_cpus": os.cpu_count(),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the run, copy 256 MiB three times (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported by this build "
              "(the path is single-GPU; the sharding design is described in the docs).", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_nf4_quantized_08_amd import lib

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib.load()
    g = torch.Generator(device=dev)
    g.manual_seed(1234)

    def randn(shape, std):
        return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std).to(torch.bfloat16)

    Ws = [torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * 0.02 for _ in range(SLOTS)]
    Xd = randn((M_DEC, K), 1.0)
    Xp = randn((M_PRE, K), 1.0)
    A = randn((R, K), 0.01)
    B = randn((N, R), 0.01)
    dY = randn((M_PRE, N), 1.0)
    n = N * K
    slots = []
    for i in range(SLOTS):
        codes = torch.empty(n // 2, dtype=torch.uint8, device=dev)
        absmax = torch.empty(n // 64, dtype=torch.float32, device=dev)
        aq = torch.empty(n // 64, dtype=torch.uint8, device=dev)
        s2 = torch.empty((n // 64 + 255) // 256, dtype=torch.float32, device=dev)
        slots.append(lib.NF4Weight(codes, absmax, aq, s2, N, K))
    deq = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    Yd = torch.empty((M_DEC, N), dtype=torch.bfloat16, device=dev)
    Yp = torch.empty((M_PRE, N), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M_PRE, K), dtype=torch.bfloat16, device=dev)
    dA = torch.empty((R, K), dtype=torch.bfloat16, device=dev)
    dB = torch.empty((N, R), dtype=torch.bfloat16, device=dev)
    ws_dec = lib.workspace(lib.QN_OP_FWD, M_DEC, N, K, R, dev)
    ws_pre = lib.workspace(lib.QN_OP_FWD, M_PRE, N, K, R, dev)
    ws_bwd = lib.workspace(lib.QN_OP_BWD, M_PRE, N, K, R, dev)

    def quantize(i):
        w = slots[i % SLOTS]
        lib.nf4_quantize(Ws[i % SLOTS], codes=w.codes, absmax=w.absmax)
        lib.nf4_double_quant(w.absmax, absmax_q=w.absmax_q, scale2=w.scale2)

    def step(i, ev=None):
        def mark(k):
            if ev is not None:
                ev[k].record()
        mark(0)
        quantize(i)
        mark(1)
        w = slots[(i + 2) % SLOTS]
        lib.nf4_dequant(w, "bf16", out=deq)
        mark(2)
        lib.qlora_linear_fwd(Xd, w, A, B, ALPHA, Y=Yd, ws=ws_dec)
        mark(3)
        lib.qlora_linear_fwd(Xp, w, A, B, ALPHA, Y=Yp, ws=ws_pre)
        mark(4)
        lib.qlora_linear_bwd(dY, Xp, w, A, B, ALPHA, out=(dX, dA, dB), ws=ws_bwd)
        mark(5)

    for i in range(SLOTS):
        quantize(i)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # One graph per slot phase (the step reads/writes slot-dependent buffers).
    graphs = []
    cap = torch.cuda.Stream()
    for ph in range(SLOTS):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            step(ph)
        graphs.append(g)
    for i in range(args.warmup):
        graphs[i % SLOTS].replay()
    torch.cuda.synchronize()

    # ---- timed region: graph replays
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[(args.warmup + i) % SLOTS].replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    # ---- each stage alone: a graph of STAGE_REPS back-to-back calls (rotating
    # weight slots), replayed; HIP events around the replays on the capture stream
    def stage_fns(i):
        w = slots[(i + 2) % SLOTS]
        return {
            "quantize": lambda: lib.nf4_quantize(Ws[i % SLOTS], codes=slots[i % SLOTS].codes,
                                                 absmax=slots[i % SLOTS].absmax),
            "double_quant": lambda: lib.nf4_double_quant(slots[i % SLOTS].absmax, absmax_q=slots[i % SLOTS].absmax_q,
                                                         scale2=slots[i % SLOTS].scale2),
            "dequant": lambda: lib.nf4_dequant(w, "bf16", out=deq),
            "fwd_decode": lambda: lib.qlora_linear_fwd(Xd, w, A, B, ALPHA, Y=Yd, ws=ws_dec),
            "fwd_prefill": lambda: lib.qlora_linear_fwd(Xp, w, A, B, ALPHA, Y=Yp, ws=ws_pre),
            "bwd": lambda: lib.qlora_linear_bwd(dY, Xp, w, A, B, ALPHA, out=(dX, dA, dB), ws=ws_bwd),
        }
    # Bandwidth-bound stages cycle through more distinct buffers than the 256 MB
    # Infinity Cache holds: 8 fp32 weights (512 MiB) to quantise, 64 NF4 weights
    # (553 MB) to dequantise or multiply at M = 1.
    wq_pool = [Ws[j % SLOTS].clone() for j in range(8)]
    nf_pool = [lib.NF4Weight(slots[j % SLOTS].codes.clone(), slots[j % SLOTS].absmax.clone(),
                             slots[j % SLOTS].absmax_q.clone(), slots[j % SLOTS].scale2.clone(), N, K)
               for j in range(64)]
    pool_fns = {
        "quantize": (8, lambda i: lib.nf4_quantize(wq_pool[i], codes=slots[i % SLOTS].codes,
                                                   absmax=slots[i % SLOTS].absmax)),
        "dequant": (64, lambda i: lib.nf4_dequant(nf_pool[i], "bf16", out=deq)),
        "fwd_decode": (64, lambda i: lib.qlora_linear_fwd(Xd, nf_pool[i], A, B, ALPHA, Y=Yd, ws=ws_dec)),
    }
    stage_us = {}
    for name in stage_fns(0):
        reps, fn = pool_fns.get(name, (STAGE_REPS, None))
        sg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(sg, stream=cap):
            for i in range(reps):
                if fn is None:
                    stage_fns(i)[name]()
                else:
                    fn(i)
        for _ in range(2):
            sg.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(cap):
            e0.record(cap)
            for _ in range(STAGE_REPLAYS):
                sg.replay()
            e1.record(cap)
        torch.cuda.synchronize()
        stage_us[name] = e0.elapsed_time(e1) * 1e3 / (STAGE_REPLAYS * reps)
        del sg
    del wq_pool, nf_pool
    # Decode on the 70B-shaped gate projection (28672 x 8192, r = 64), where the
    # GEMV is bound by weight bandwidth rather than by launch latency: three
    # distinct NF4 weights (3 x 121 MB, more than the Infinity Cache) in turn.
    N70, K70, R70 = 28672, 8192, 64
    g70 = torch.Generator(device=dev)
    g70.manual_seed(70)
    w70 = []
    for _ in range(3):
        src = (torch.randn((N70, K70), generator=g70, device=dev) * 0.015).to(torch.bfloat16)
        w70.append(lib.quantize_weight(src))
        del src
    A70 = (torch.randn((R70, K70), generator=g70, device=dev) * 0.01).to(torch.bfloat16)
    B70 = (torch.randn((N70, R70), generator=g70, device=dev) * 0.01).to(torch.bfloat16)
    X70 = torch.randn((1, K70), generator=g70, device=dev).to(torch.bfloat16)
    Y70 = torch.empty((1, N70), dtype=torch.bfloat16, device=dev)
    ws70 = lib.workspace(lib.QN_OP_FWD, 1, N70, K70, R70, dev)
    sg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(sg, stream=cap):
        for i in range(6):
            lib.qlora_linear_fwd(X70, w70[i % 3], A70, B70, 2.0 * R70, Y=Y70, ws=ws70)
    for _ in range(2):
        sg.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(cap):
        e0.record(cap)
        for _ in range(STAGE_REPLAYS):
            sg.replay()
        e1.record(cap)
    torch.cuda.synchronize()
    dec70_us = e0.elapsed_time(e1) * 1e3 / (STAGE_REPLAYS * 6)
    nb70 = N70 * K70 // 64
    dec70_bytes = N70 * K70 // 2 + nb70 + 4 * ((nb70 + 255) // 256)
    del sg, w70, A70, B70, X70, Y70, ws70
    # Bulk round trip: 7.62e9 weights streamed as 4096 x 4096 bf16 tiles
    # (N(0, 0.02)) through NF4 quantisation, double quantisation and bf16
    # dequantisation.  Sixteen distinct tiles (537 MB of source, more than the
    # Infinity Cache) stand in for the stream; the sweep time is the per-tile
    # time times the number of tiles.
    SWEEP_WEIGHTS, TILE = 7.62e9, 4096 * 4096
    g_sw = torch.Generator(device=dev)
    g_sw.manual_seed(762)
    tiles = [(torch.randn((4096, 4096), generator=g_sw, device=dev) * 0.02).to(torch.bfloat16) for _ in range(16)]
    sw = [lib.quantize_weight(tiles[j]) for j in range(2)]
    sw_out = torch.empty((4096, 4096), dtype=torch.bfloat16, device=dev)
    sg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(sg, stream=cap):
        for j in range(16):
            w = sw[j % 2]
            lib.nf4_quantize(tiles[j], codes=w.codes, absmax=w.absmax)
            lib.nf4_double_quant(w.absmax, absmax_q=w.absmax_q, scale2=w.scale2)
            lib.nf4_dequant(w, "bf16", out=sw_out)
    for _ in range(2):
        sg.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(cap):
        e0.record(cap)
        for _ in range(STAGE_REPLAYS):
            sg.replay()
        e1.record(cap)
    torch.cuda.synchronize()
    tile_us = e0.elapsed_time(e1) * 1e3 / (STAGE_REPLAYS * 16)
    nb_t = TILE // 64
    # bytes per tile: quantise (bf16 in, codes + fp32 scales out), double quant
    # (fp32 scales in, 8-bit scales + steps out), dequant (codes + 8-bit scales +
    # steps in, bf16 out)
    tile_bytes = (2 * TILE + TILE // 2 + 4 * nb_t) + (4 * nb_t + nb_t + 4 * (nb_t // 256)) + \
                 (TILE // 2 + nb_t + 4 * (nb_t // 256) + 2 * TILE)
    sweep = {
        "tile_round_trip_us": round(tile_us, 2),
        "round_trip_GBps": round(tile_bytes / (tile_us * 1e-6) / 1e9, 1),
        "sweep_7.62e9_weights_ms": round(SWEEP_WEIGHTS / TILE * tile_us * 1e-3, 2),
        "stored_bits_per_param": round((TILE // 2 + nb_t + 4 * (nb_t // 256)) * 8 / TILE, 6),
    }
    del sg, tiles, sw, sw_out
    layers = {"qwen2.5_7b": layer_times(lib, dev, cap, QWEN_LINEARS, 16, 4096, bwd=True),
              "70b": layer_times(lib, dev, cap, L70B_LINEARS, 64, 4096, bwd=False)}
    # the quantise stages overwrote slot contents with the same values; restore order
    for i in range(SLOTS):
        quantize(i)
    torch.cuda.synchronize()

    # ---- traced eager pass over the same steps: per-kernel durations
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    lib.trace_enable(True)
    torch.cuda.synchronize()
    te0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    te1 = time.perf_counter()
    trace = lib.trace_read()
    lib.trace_enable(False)
    stage_ms = {k: 0.0 for k in ("quantize+dq", "dequant", "fwd_decode", "fwd_prefill", "bwd")}
    names = list(stage_ms)
    for e in evs:
        for j in range(5):
            stage_ms[names[j]] += e[j].elapsed_time(e[j + 1]) / args.steps
    kern = {}
    for kind, ms in trace:
        kern.setdefault(kind, []).append(ms)
    kern_avg = {k: sum(v) / len(v) for k, v in kern.items()}
    kern_per_step = {k: sum(v) / args.steps for k, v in kern.items()}

    s = sizes()
    flops_step = s["fwd_flops"] + s["bwd_flops"] + s["gemv_flops"]
    value = flops_step / (ms_step * 1e-3) / 1e12

    work = {  # algorithmic work per launch, and its roofline
        "quantize": (s["quantize_bytes"], "hbm"),
        "double_quant": (s["dq_bytes"], "hbm"),
        "dequant": (s["dequant_bytes"], "hbm"),
        "gemv": (s["gemv_all_bytes"], "hbm"),
        "gemm_fwd": (s["fwd_gemm_kernel_flops"], "mfma"),
        "gemm_dx": (s["dx_gemm_kernel_flops"], "mfma"),
        "lowrank": ((s["lowrank_fwd_bytes"] + s["lowrank_bwd_bytes"]) // 2, "hbm"),
        "gemm_db": (s["colred_bytes"], "hbm"),
    }

    def roof(kind):
        amount, bound = work[kind]
        avg = kern_avg[kind]
        if bound == "hbm":
            ach = amount / (avg * 1e-3) / 1e9
            return {"kernel": kind, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": traffic(kind),
                    "avg_ms": round(avg, 5), "work_per_launch": amount}
        ach = amount / (avg * 1e-3) / 1e12
        return {"kernel": kind, "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic(kind),
                "avg_ms": round(avg, 5), "work_per_launch": amount}

    dominant = max((k for k in kern_per_step if k in work), key=lambda k: kern_per_step[k])
    stages = {
        "stage_us_graph": {k: round(v, 2) for k, v in stage_us.items()},
        "prefill_fwd_call_TFLOPs": round(s["fwd_flops"] / (stage_us["fwd_prefill"] * 1e-6) / 1e12, 1),
        "prefill_fwd_gemm_kernel_TFLOPs": round(s["fwd_gemm_kernel_flops"] / (kern_avg["gemm_fwd"] * 1e-3) / 1e12, 1),
        "bwd_call_TFLOPs": round(s["bwd_flops"] / (stage_us["bwd"] * 1e-6) / 1e12, 1),
        "decode_call_weight_GBps": round(s["gemv_weight_bytes"] / (stage_us["fwd_decode"] * 1e-6) / 1e9, 1),
        "decode_call_all_GBps": round(s["gemv_all_bytes"] / (stage_us["fwd_decode"] * 1e-6) / 1e9, 1),
        "bulk_round_trip_bf16_tiles": sweep,
        "layers_M4096": layers,
        "decode_70b_gate_call_us": round(dec70_us, 2),
        "decode_70b_gate_call_weight_GBps": round(dec70_bytes / (dec70_us * 1e-6) / 1e9, 1),
        "quantize_GBps": round(s["quantize_bytes"] / (stage_us["quantize"] * 1e-6) / 1e9, 1),
        "double_quant_GBps": round(s["dq_bytes"] / (stage_us["double_quant"] * 1e-6) / 1e9, 1),
        "dequant_GBps": round(s["dequant_bytes"] / (stage_us["dequant"] * 1e-6) / 1e9, 1),
        "stage_ms_eager_traced": {k: round(v, 4) for k, v in stage_ms.items()},
        "eager_traced_ms_per_step": round((te1 - te0) * 1e3 / args.steps, 4),
        "kernel_avg_ms": {k: round(v, 5) for k, v in kern_avg.items()},
        "kernel_rooflines": {k: roof(k) for k in work if k in kern_avg},
    }
    out = {
        "metric": "NF4 dequant-GEMM TFLOP/s (prefill), weight GB/s (decode GEMV), quantize GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "single 4096x4096 projection: NF4 bs64 + double quant bs256, LoRA r=16 alpha=32, "
                               "decode M=1 and prefill M=2048 forward, backward at M=2048, fp32 weight source",
                   "N": N, "K": K, "r": R, "alpha": ALPHA, "M_decode": M_DEC, "M_prefill": M_PRE},
        "metrics": {
            "prefill_dequant_gemm_TFLOPs": stages["prefill_fwd_gemm_kernel_TFLOPs"],
            "decode_gemv_weight_GBps": stages["decode_call_weight_GBps"],
            "decode_gemv_weight_GBps_70b_gate": stages["decode_70b_gate_call_weight_GBps"],
            "quantize_GBps": stages["quantize_GBps"],
        },
        "roofline": roof(dominant),
        "stages": stages,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("copy calibration: 3 x 268435456 B read + written", file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
