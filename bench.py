"""Throughput of the NF4 / QLoRA-linear hot path on one MI355X.

Headline workload: the 70B-shaped transformer layer (hidden 8192; q, o 8192x8192,
k, v 1024x8192, gate, up 28672x8192, down 8192x28672), each weight
N(0, 0.015^2) fp32 with 0.1 % of its entries (seeded Bernoulli positions) x10,
quantised once to NF4 (blocks of 64) with double quantisation (groups of 256)
before the timed region -- the method quantises while loading; LoRA r = 64,
alpha = 128 on every linear.

One step = that configuration's pass over all seven linears:

  decode forward, X: 1 x K per linear                qlora_linear_fwd (M = 1)
  prefill forward, X: 4096 x K per linear            qlora_linear_fwd (M = 4096)

The step is captured once into a HIP graph and the timed region replays it.
`value` = the step's algorithmic contraction work (2 per multiply-add over
X W^T, X A^T and H B^T; the expansion of the codes is not counted) divided by
the step time: the dequant-GEMM TFLOP/s of the layer, whole-step.

`metrics` (each timed alone, graph-replayed):
  prefill_dequant_gemm_TFLOPs   the layer's M = 4096 forward alone
  decode_gemv_weight_GBps       the layer's M = 1 forward alone (441 MB of NF4
                                weights, more than the 256 MB Infinity Cache)
  quantize_GBps                 nf4_quantize on 4096 x 4096 bf16 tiles of the
                                bulk sweep (7.62e9 weights)
`stages` holds the rest of the path, each on its own configuration: the
single 4096x4096 projection (quantise from fp32, double quant, dequant, decode,
prefill forward and backward), the Qwen2.5-7B-shaped layer at M = 4096 forward
and backward per linear, the bulk quantise / double-quant / dequant round trip
with its error and stored bits per weight, the tiny configuration's call times,
and the 70B layer's dequantisation error with and without double quantisation.

A second, eager pass over the same step enables the library's kernel trace:
HIP events recorded around each call's dominant kernel on its own launch
stream.  The `roofline` object is the dominant kernel of the step (the forward
dequant-GEMM): algorithmic FLOPs of its launches over their summed durations.
`roofline.traffic` is the HBM bytes per launch from rocprofv3 FETCH_SIZE and
WRITE_SIZE counters (table `TRAFFIC`, each counter scaled by what it reads for
a plain copy of known size, taken with `--copy-calibration`); null when no such
measurement exists for the kernel source as it is now.  `cpu_baseline` times
the CPU oracle on a bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3
STAGE_REPS, STAGE_REPLAYS = 8, 5
CSRC = os.path.join(ROOT, "bit_nf4_quantized_08_amd", "csrc")
KERNEL_SOURCE = {
    "quantize": "k_codec.hip", "double_quant": "k_codec.hip", "dequant": "k_codec.hip",
    "gemv": "k_linear.hip", "gemm_fwd": "k_qgemm.hip", "gemm_dx": "k_qgemm.hip",
    "lowrank": "k_lowrank.hip", "gemm_db": "k_lowrank.hip", "gemm_da": "k_lowrank.hip",
}
# Measured memory-side bytes per launch: rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE
# (KiB per dispatch), each scaled by the ratio of known bytes to counted bytes for a
# 256 MiB copy in the same run, averaged over the step's four calls of the
# kernel (a call's launches counted together).  The counters see the traffic between the L2 caches and the memory
# fabric (reads served by the Infinity Cache included), an upper bound on HBM
# bytes.  Keyed by kernel and workload; `sha256` is that of the kernel's source
# file and qn_device.h when the counters were taken.
TRAFFIC = {
    "gemm_fwd_70b": {"bytes": 1565569317, "sha256": "eeece9299dab90e57c0d8c85d8c243062b22dc01db76f699f6f807421ae217ea"},
    "lowrank_70b": {"bytes": 176664927, "sha256": "a9720ed64701ca58a3adf8b5f53627d51383e3fd25feb52c5caef37c5c1ca6bb"},
    "gemv_70b": {"bytes": 114969601, "sha256": "a5da0adfb8a87a342062662a46fde1812682acb87b6815a04b93989080b3022b"},
}

# The configurations (N, K) of the linear layers.
L70B = {"q": (8192, 8192), "k": (1024, 8192), "v": (1024, 8192), "o": (8192, 8192),
        "gate": (28672, 8192), "up": (28672, 8192), "down": (8192, 28672)}
R70, ALPHA70, M70_PRE, M70_DEC, W70_STD = 64, 128.0, 4096, 1, 0.015
QWEN = {"q": (3584, 3584), "k": (512, 3584), "v": (512, 3584), "o": (3584, 3584),
        "gate": (18944, 3584), "up": (18944, 3584), "down": (3584, 18944)}
RQ, ALPHAQ, MQ = 16, 32.0, 4096
N2, K2, R2, ALPHA2, M2_DEC, M2_PRE = 4096, 4096, 16, 32.0, 1, 2048


def source_sha(kind):
    h = hashlib.sha256()
    for f in (KERNEL_SOURCE[kind], "qn_device.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic(key, kind):
    t = TRAFFIC.get(key)
    if t is None or t["sha256"] != source_sha(kind):
        return None
    return t["bytes"]


def nf4_bytes(N, K):
    """Stored bytes of one NF4 weight with double quantisation."""
    nb = N * K // 64
    return N * K // 2 + nb + 4 * ((nb + 255) // 256)


def fwd_flops(M, N, K, r):
    return 2 * M * N * K + 2 * M * K * r + 2 * M * r * N


def bwd_flops(M, N, K, r):
    return 2 * M * N * K + 4 * M * N * r + 4 * M * r * K


def lscpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def graph_time_us(torch, stream, fn, replays=STAGE_REPLAYS, calls=1):
    """Capture fn() into a graph on `stream`, replay twice untimed, then time
    `replays` replays with HIP events on the same stream; microseconds per call."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (replays * calls)
    del g
    return us


# ------------------------------------------------------------------ workloads
class Layer:
    """All linears of one layer on the device: NF4 weights with double
    quantisation, activations, adapters, outputs and workspaces."""

    def __init__(self, torch, lib, dev, linears, r, w_std, M_list, seed, outliers=False, bwd_M=None,
                 quality=False):
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        rnd = lambda shape, std: (torch.randn(shape, generator=g, device=dev) * std).to(torch.bfloat16)
        self.r, self.alpha, self.items = r, 2.0 * r, []
        sq_err = {"dq": 0.0, "fp32_scales": 0.0}
        sq_ref = 0.0
        for name, (N, K) in linears.items():
            W = torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * w_std
            if outliers:
                mask = torch.rand((N, K), generator=g, device=dev) < 0.001
                W = torch.where(mask, W * 10.0, W)
                del mask
            w = lib.quantize_weight(W)
            if quality:
                for key, dq in (("dq", True), ("fp32_scales", False)):
                    d = lib.nf4_dequant(w, "f32", use_double_quant=dq)
                    sq_err[key] += float(((d.double() - W.double()) ** 2).sum())
                    del d
                sq_ref += float((W.double() ** 2).sum())
            del W
            it = dict(name=name, N=N, K=K, w=w, A=rnd((r, K), 0.01), B=rnd((N, r), 0.01), X={}, Y={}, ws={})
            for M in M_list:
                it["X"][M] = rnd((M, K), 1.0)
                it["Y"][M] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                it["ws"][M] = lib.workspace(lib.QN_OP_FWD, M, N, K, r, dev)
            if bwd_M is not None:
                M = bwd_M
                it.update(dY=rnd((M, N), 1.0), dX=torch.empty((M, K), dtype=torch.bfloat16, device=dev),
                          dA=torch.empty((r, K), dtype=torch.bfloat16, device=dev),
                          dB=torch.empty((N, r), dtype=torch.bfloat16, device=dev),
                          H=torch.empty((M, r), dtype=torch.float32, device=dev),
                          wsb=lib.workspace(lib.QN_OP_BWD, M, N, K, r, dev))
            self.items.append(it)
        torch.cuda.synchronize()
        self.quality = None
        if quality:
            self.quality = {k: (v / sq_ref) ** 0.5 for k, v in sq_err.items()}

    def groups(self, lib, M, partition):
        """FwdGroup objects (one grouped call each) over the named linears."""
        by = {it["name"]: it for it in self.items}
        return [lib.FwdGroup([(by[n]["X"][M], by[n]["w"], by[n]["A"], by[n]["B"], self.alpha, by[n]["Y"][M], None)
                              for n in part]) for part in partition]

    def fwd(self, lib, M, items=None, want_H=False):
        for it in (items or self.items):
            lib.qlora_linear_fwd(it["X"][M], it["w"], it["A"], it["B"], self.alpha, Y=it["Y"][M], ws=it["ws"][M],
                                 H=it["H"] if want_H else None)

    def bwd(self, lib, M, items=None):
        for it in (items or self.items):
            lib.qlora_linear_bwd(it["dY"], it["X"][M], it["w"], it["A"], it["B"], self.alpha,
                                 out=(it["dX"], it["dA"], it["dB"]), ws=it["wsb"], H=it["H"])

    def flops(self, M, kind="fwd", items=None):
        f = fwd_flops if kind == "fwd" else bwd_flops
        return sum(f(M, it["N"], it["K"], self.r) for it in (items or self.items))

    def weight_bytes(self):
        return sum(nf4_bytes(it["N"], it["K"]) for it in self.items)


# ------------------------------------------------------------------ CPU oracle
def cpu_baseline():
    """The CPU oracle, as it stands, on bounded samples of the same workloads.

    `value` (the headline unit, TFLOP/s): one linear of the 70B-shaped layer
    (q, 8192 x 8192) on 256 token rows -- the oracle's dequantisation of the NF4
    weight to bf16 values (one core, numpy) plus its fp64 forward (all BLAS
    threads); quantisation happens before the timer, as on the GPU.  Also reported
    (not the headline): codec GB/s on the tiny configuration, the 4096 x 4096
    weight and 8 bulk tiles; fp64 contraction GFLOP/s on the tiny configuration,
    the 4096 x 4096 projection (forward M = 2048 and backward) and 256-row subsets
    of the Qwen2.5-7B- and 70B-shaped layers' linears (contraction only: its cost
    does not depend on the weight's values, so a Gaussian bf16 matrix stands in
    for W_hat there)."""
    import numpy as np
    import oracle
    from bit_nf4_quantized_08_amd import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    t_all = time.perf_counter()
    bf = lambda shape, std, seed: synth.bf16_values(synth.to_bf16(synth.gaussian(shape, std, seed)))
    out = {"kind": "oracle", "unit": "TFLOP/s", "cores": int(blas_threads), "host_cpus": os.cpu_count(),
           "cpu_model": lscpu_model()}

    def codec_rate(W):
        n = W.size
        t0 = time.perf_counter()
        p, a, _ = oracle.quantize(W)
        k, st = oracle.double_quant(a)
        oracle.dequant_bf16_weight(p, W.shape[0], W.shape[1], oracle.dq_absmax(k, st))
        dt = time.perf_counter() - t0
        in_b = 4 if W.dtype == np.float32 else 2
        nb = (n + 63) // 64
        byts = (in_b * n + n // 2 + 4 * nb) + (5 * nb + 4 * ((nb + 255) // 256)) + (n // 2 + nb + 2 * n)
        return byts, dt

    # headline sample: 70B q projection, 256 rows
    N, K = L70B["q"]
    Wq = synth.with_outliers(synth.gaussian((N, K), W70_STD, synth.SEED_W), 0.001, 10.0)
    p, a, _ = oracle.quantize(Wq)
    k, st = oracle.double_quant(a)
    X = bf((256, K), 1.0, synth.SEED_X)
    A, B = bf((R70, K), 0.01, synth.SEED_A), bf((N, R70), 0.01, synth.SEED_B)
    t0 = time.perf_counter()
    Wh = oracle.dequant_bf16_weight(p, N, K, oracle.dq_absmax(k, st))
    t1 = time.perf_counter()
    oracle.forward(X, Wh, A, B, ALPHA70)
    t2 = time.perf_counter()
    fl = fwd_flops(256, N, K, R70)
    out["value"] = fl / (t2 - t0) / 1e12
    out["sample"] = (f"70B-shaped q projection (8192x8192, NF4 + double quant, r=64) forward of 256 token rows: "
                     f"oracle bf16 dequantisation {t1 - t0:.2f} s on 1 core + fp64 forward {t2 - t1:.2f} s on "
                     f"{blas_threads} BLAS threads; value = that sample's contraction FLOPs / its time")
    del Wq, p, a, k, st, Wh
    # codec GB/s
    codec = {}
    tiny = synth.tiny_inputs()
    b, dt = codec_rate(tiny["W"])
    codec["tiny_256x512_fp32"] = round(b / dt / 1e9, 4)
    b, dt = codec_rate(synth.gaussian((N2, K2), 0.02, synth.SEED_W))
    codec["proj4096_fp32"] = round(b / dt / 1e9, 4)
    tb, tt = 0, 0.0
    for t in range(8):
        W = bf((4096, 4096), 0.02, synth.SEED_BULK0 + t)   # bf16 values, widened exactly
        b, dt = codec_rate(W)
        tb += b - 2 * W.size    # bf16 source: 2 bytes in, not 4
        tt += dt
    codec["bulk_8_tiles_bf16"] = round(tb / tt / 1e9, 4)
    out["codec_GBps_1core"] = codec
    # fp64 contractions
    con = {}

    def con_rate(M, N, K, r, bwd=True, reps=1):
        X, A, B = bf((M, K), 1.0, 2), bf((r, K), 0.01, 3), bf((N, r), 0.01, 4)
        Wh = bf((N, K), 0.02, 1)
        G = bf((M, N), 1.0, 5) if bwd else None
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.forward(X, Wh, A, B, 2.0 * r)
            if bwd:
                oracle.backward(G, X, Wh, A, B, 2.0 * r)
        dt = time.perf_counter() - t0
        return reps * (fwd_flops(M, N, K, r) + (bwd_flops(M, N, K, r) if bwd else 0)), dt

    f, dt = con_rate(4, 256, 512, 8, reps=50)
    con["tiny_fwd_bwd"] = round(f / dt / 1e9, 3)
    f, dt = con_rate(M2_PRE, N2, K2, R2)
    con["proj4096_M2048_fwd_bwd"] = round(f / dt / 1e9, 3)
    for tag, lin, r, bwd in (("qwen7b_layer_256rows_fwd_bwd", QWEN, RQ, True), ("70b_layer_256rows_fwd", L70B, R70, False)):
        tf, tt = 0, 0.0
        for (n_, k_) in lin.values():
            f, dt = con_rate(256, n_, k_, r, bwd=bwd)
            tf += f
            tt += dt
        con[tag] = round(tf / tt / 1e9, 3)
    out["contraction_GFLOPs_fp64"] = con
    out["seconds"] = round(time.perf_counter() - t_all, 1)
    return out


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stages", action="store_true", help="headline step only (for profiling runs)")
    ap.add_argument("--bulk-only", action="store_true",
                    help="only the bulk round trip over 4096x4096 bf16 tiles, printed as one JSON line "
                         "(for profiling the codec kernels)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the run, copy 256 MiB three times (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: this build runs the path on "
              "a single GPU (how it would shard is described in the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_nf4_quantized_08_amd import lib

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib.load()
    cap = torch.cuda.Stream()
    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)
    if args.bulk_only:
        print(json.dumps({"bulk_round_trip_bf16_tiles": bulk_stage(torch, lib, dev, cap, log)}), flush=True)
        return

    # ---------------- headline: the 70B-shaped layer
    log("70B layer: quantising 7 weights")
    L = Layer(torch, lib, dev, L70B, R70, W70_STD, [M70_DEC, M70_PRE], seed=70, outliers=True, quality=True)

    # Grouped calls in the order a layer's data allows: q, k, v read the same
    # normalised hidden state; o reads the attention output; gate and up read
    # the same normalised hidden state; down reads act(gate) * up.
    dep = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
    dec_groups = L.groups(lib, M70_DEC, dep)
    pre_groups = L.groups(lib, M70_PRE, dep)
    all7 = L.groups(lib, M70_PRE, [tuple(L70B)])

    def step():
        for grp in dec_groups:
            grp.run()
        for grp in pre_groups:
            grp.run()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    del g
    ms_step = (t1 - t0) * 1e3 / args.steps
    step_flops = L.flops(M70_DEC) + L.flops(M70_PRE)
    value = step_flops / (ms_step * 1e-3) / 1e12

    # the two halves of the step alone
    pre_us = graph_time_us(torch, cap, lambda: [grp.run() for grp in pre_groups])
    dec_us = graph_time_us(torch, cap, lambda: [grp.run() for grp in dec_groups], replays=20)

    # kernel trace over one eager step
    # One untraced step first: while the GPU runs its M = 4096 GEMMs the host
    # enqueues the traced step, whose kernels then run back to back, so that
    # the trace events bracket the kernels rather than host launch gaps.
    torch.cuda.synchronize()
    step()
    lib.trace_enable(True)
    step()
    torch.cuda.synchronize()
    trace = lib.trace_read()
    lib.trace_enable(False)
    kern = {}
    for kind, ms in trace:
        kern.setdefault(kind, []).append(ms)
    gemm = kern["gemm_fwd"]
    gemm_flops = sum(2 * M70_PRE * it["N"] * it["K"] + 2 * M70_PRE * R70 * it["N"] for it in L.items)
    ach = gemm_flops / (sum(gemm) * 1e-3) / 1e12
    roofline = {"kernel": "gemm_fwd", "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic("gemm_fwd_70b", "gemm_fwd"),
                "launches": len(gemm), "avg_ms": round(sum(gemm) / len(gemm), 5),
                "launch_ms": [round(x, 5) for x in gemm],
                "work_per_launch": gemm_flops // len(gemm),
                "launch_flops": [sum(2 * M70_PRE * L70B[n][0] * L70B[n][1] + 2 * M70_PRE * R70 * L70B[n][0] for n in part)
                                 for part in dep],
                "note": "grouped calls q,k,v | o | gate,up | down at M = 4096, one entry per call (the q,k,v "
                        "call runs q on 256x256 tiles and k, v on 256x128 tiles, two launches traced together); "
                        "work = 2MNK + 2MrN over the linears of each call (the X A^T product runs in the low-rank "
                        "kernel)"}
    gemv = kern.get("gemv", [])
    gemv_bytes = sum(nf4_bytes(it["N"], it["K"]) + 2 * it["K"] + 2 * it["N"] + 2 * R70 * it["K"] for it in L.items)
    gemv_roof = None
    if gemv:
        a = gemv_bytes / (sum(gemv) * 1e-3) / 1e9
        gemv_roof = {"kernel": "gemv", "bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(a / PEAK_HBM_GBPS, 4), "traffic": traffic("gemv_70b", "gemv"),
                     "launches": len(gemv), "avg_ms": round(sum(gemv) / len(gemv), 5),
                     "note": "the streaming kernel alone (its epilogue launch excluded); bytes = NF4 weights + "
                             "x + y + A (read for the H partials)"}
    lowr = kern.get("lowrank", [])
    lowrank_roof = None
    if lowr:
        # per problem: X read once, A read, H written fp32 and bf16(s H)
        lr_bytes = sum(2 * M70_PRE * it["K"] + 2 * R70 * it["K"] + 6 * M70_PRE * R70 for it in L.items)
        a = lr_bytes / (sum(lowr) * 1e-3) / 1e9
        lowrank_roof = {"kernel": "lowrank", "bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBPS,
                        "unit": "GB/s", "frac": round(a / PEAK_HBM_GBPS, 4),
                        "traffic": traffic("lowrank_70b", "lowrank"), "launches": len(lowr),
                        "launch_ms": [round(x, 5) for x in lowr],
                        "note": "H = X A^T of the prefill step, one launch per dependency group (its finishing "
                                "launch excluded); bytes = X, A and H per linear"}
    flops_pre = sum(fwd_flops(M70_PRE, n_, k_, R70) for n_, k_ in L70B.values())
    weight_bytes = L.weight_bytes()
    layer_stage = {}
    if not args.no_stages:
        layer_stage = layer_extras(torch, lib, dev, cap, L, pre_groups, all7, log, flops_pre, weight_bytes, pre_us,
                                   dec_us)
    quality = L.quality
    del L
    torch.cuda.empty_cache()

    stages = {"70b_layer": {"prefill_M4096_us": round(pre_us, 1),
                            "prefill_M4096_TFLOPs": round(flops_pre / pre_us / 1e6, 1),
                            "decode_M1_us": round(dec_us, 2),
                            "decode_M1_weight_GBps": round(weight_bytes / dec_us / 1e3, 1),
                            "dequant_rel_rmse": {k: round(v, 6) for k, v in quality.items()},
                            "gemv_roofline": gemv_roof,
                            "lowrank_roofline": lowrank_roof}}
    stages["70b_layer"].update(layer_stage)
    metrics = {"prefill_dequant_gemm_TFLOPs": round(flops_pre / pre_us / 1e6, 1),
               "decode_gemv_weight_GBps": round(weight_bytes / dec_us / 1e3, 1)}

    if not args.no_stages:
        stages.update(other_stages(torch, lib, dev, cap, log))
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
        "config": {"workload": "70B-shaped layer: q/o 8192x8192, k/v 1024x8192, gate/up 28672x8192, down "
                               "8192x28672; W ~ N(0, 0.015^2) with 0.1% outliers x10 in NF4 bs64 + double quant "
                               "bs256; LoRA r=64 alpha=128; decode M=1 and prefill M=4096 forward over all 7 linears",
                   "hidden": 8192, "r": R70, "alpha": ALPHA70, "M_decode": M70_DEC, "M_prefill": M70_PRE},
    }
    if "bulk_round_trip_bf16_tiles" in stages:
        metrics["quantize_GBps"] = stages["bulk_round_trip_bf16_tiles"]["quantize_GBps"]
    out["metrics"] = metrics
    out["roofline"] = roofline
    out["stages"] = stages
    if not args.no_cpu_baseline:
        log("cpu baseline")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("copy calibration: 3 x 268435456 B read + written", file=sys.stderr, flush=True)



def layer_extras(torch, lib, dev, cap, L, pre_groups, all7, log, flops_pre, weight_bytes, pre_us, dec_us):
    """The 70B layer's other timings: the forward as 7 single calls and as one
    call over all 7 linears, each forward tiling, each linear alone, the merge
    of all adapters into bf16 weights and one 8-bit AdamW step over them."""
    log("70B layer: single calls, tilings, per linear, merge, AdamW")
    dec_single_us = graph_time_us(torch, cap, lambda: L.fwd(lib, M70_DEC), replays=20)
    dec_all7 = L.groups(lib, M70_DEC, [tuple(L70B)])
    dec_all7_us = graph_time_us(torch, cap, lambda: dec_all7[0].run(), replays=20)
    pre_single_us = graph_time_us(torch, cap, lambda: L.fwd(lib, M70_PRE))
    pre_all7_us = graph_time_us(torch, cap, lambda: all7[0].run())
    tilings = {}
    for v in (1, 2, 3):
        lib.set_gemm_variant(v)
        tilings[v] = graph_time_us(torch, cap, lambda: [grp.run() for grp in pre_groups])
    lib.set_gemm_variant(0)
    per_linear = {}
    for it in L.items:
        us = graph_time_us(torch, cap, lambda: L.fwd(lib, M70_PRE, [it]))
        # ten calls per graph: one small call is shorter than a graph launch
        dus = graph_time_us(torch, cap, lambda: [L.fwd(lib, M70_DEC, [it]) for _ in range(10)], replays=5, calls=10)
        per_linear[it["name"]] = {"prefill_us": round(us, 1),
                                  "prefill_TFLOPs": round(fwd_flops(M70_PRE, it["N"], it["K"], R70) / us / 1e6, 1),
                                  "decode_us": round(dus, 2),
                                  "decode_weight_GBps": round(nf4_bytes(it["N"], it["K"]) / dus / 1e3, 1)}
    # batched decode (M = 8 activation rows) on the gate projection
    gate = next(it for it in L.items if it["name"] == "gate")
    X8 = (torch.randn((8, gate["K"]), device=dev)).to(torch.bfloat16)
    Y8 = torch.empty((8, gate["N"]), dtype=torch.bfloat16, device=dev)
    ws8 = lib.workspace(lib.QN_OP_FWD, 8, gate["N"], gate["K"], R70, dev)
    gate_m8_us = graph_time_us(torch, cap, lambda: [lib.qlora_linear_fwd(X8, gate["w"], gate["A"], gate["B"], L.alpha,
                                                                         Y=Y8, ws=ws8) for _ in range(10)],
                               replays=5, calls=10)
    del X8, Y8, ws8
    # merge/export of the layer's adapters into bf16 weights (one call per linear)
    mo = {it["name"]: torch.empty((it["N"], it["K"]), dtype=torch.bfloat16, device=dev) for it in L.items}
    merge_us = graph_time_us(torch, cap, lambda: [lib.qlora_merge(it["w"], it["A"], it["B"], L.alpha, out=mo[it["name"]])
                                                  for it in L.items], replays=3)
    n_el = sum(it["N"] * it["K"] for it in L.items)
    merge_bytes = sum(nf4_bytes(it["N"], it["K"]) + 2 * it["N"] * it["K"] + 2 * R70 * (it["N"] + it["K"])
                      for it in L.items)
    merge = {"us": round(merge_us, 1), "GBps": round(merge_bytes / merge_us / 1e3, 1),
             "fma_TFLOPs": round(2 * R70 * n_el / merge_us / 1e6, 1),
             "alu_frac": round(2 * R70 * n_el / merge_us / 1e6 / PEAK_FP32_TFLOPS, 4),
             "note": "all 7 linears merged to bf16 (r = 64): r fused multiply-adds per weight, bound by the fp32 "
                     "vector rate (157.3 TFLOP/s) rather than by its bytes"}
    del mo
    # one 8-bit AdamW step over the layer's adapters (A and B of every linear)
    ad_t = [(t, t.clone(), lib.AdamW8State(t.numel(), dev)) for it in L.items for t in (it["A"], it["B"])]
    ad_n = sum(t.numel() for t, _, _ in ad_t)
    for t, gr, stt in ad_t:
        lib.adamw8_step(t, gr, stt, lr=1e-4, step=1)
    adam_us = graph_time_us(torch, cap, lambda: [lib.adamw8_step(t, gr, stt, lr=1e-4, step=2) for t, gr, stt in ad_t],
                            replays=10)
    adam_multi_us = graph_time_us(torch, cap, lambda: lib.adamw8_step_multi([t for t, _, _ in ad_t],
                                                                            [gr for _, gr, _ in ad_t],
                                                                            [stt for _, _, stt in ad_t],
                                                                            lr=1e-4, step=2), replays=10)
    ad_host = [lib.AdamW8State(t.numel(), dev, host=True) for t, _, _ in ad_t]
    lib.adamw8_step_multi([t for t, _, _ in ad_t], [gr for _, gr, _ in ad_t], ad_host, lr=1e-4, step=1)
    adam_host_us = graph_time_us(torch, cap, lambda: lib.adamw8_step_multi([t for t, _, _ in ad_t],
                                                                           [gr for _, gr, _ in ad_t], ad_host,
                                                                           lr=1e-4, step=2), replays=5)
    adam_bytes = ad_n * (2 + 2 + 2 + 2 + 1 + 1) + 2 * 2 * 4 * ((ad_n + 63) // 64)
    state_bytes = 2 * (2 * ad_n + 2 * 4 * ((ad_n + 63) // 64))   # both codes and steps, read and written
    adamw8 = {"us": round(adam_multi_us, 2), "params": ad_n, "GBps": round(adam_bytes / adam_multi_us / 1e3, 1),
              "hbm_frac": round(adam_bytes / adam_multi_us / 1e3 / PEAK_HBM_GBPS, 4),
              "per_tensor_calls_us": round(adam_us, 2),
              "host_state_us": round(adam_host_us, 1),
              "host_state_link_GBps": round(state_bytes / adam_host_us / 1e3, 1),
              "state_bytes_per_param": 2.125,
              "note": "one qn_adamw8_step_multi over the 14 tensors (A and B of the 7 linears, r = 64); "
                      "per_tensor_calls_us: 14 qn_adamw8_step calls; bytes = bf16 parameter read and written, bf16 "
                      "gradient, both 8-bit codes read and written, block steps; host_state: the same step with "
                      "the 8-bit state in pinned host memory (the paged placement), its state bytes crossing the "
                      "host link"}
    del ad_t, ad_host
    ctx = context_ceilings(torch, dev, log)
    f, w = flops_pre, weight_bytes
    ctx["nf4_prefill_over_dense_bf16"] = round(f / pre_us / 1e6 / ctx["hipblaslt_bf16_layer_M4096_TFLOPs"], 3)
    ctx["nf4_decode_speedup_over_dense_bf16"] = round(ctx["dense_bf16_decode_M1_layer_us"] / dec_us, 2)
    return {"context_ceilings": ctx,
            "prefill_M4096_single_calls_TFLOPs": round(f / pre_single_us / 1e6, 1),
            "prefill_M4096_one_call_all7_TFLOPs": round(f / pre_all7_us / 1e6, 1),
            "prefill_M4096_TFLOPs_by_tiling": {
                "256x128": round(f / tilings[1] / 1e6, 1), "256x256_8waves": round(f / tilings[2] / 1e6, 1),
                "256x256_4waves": round(f / tilings[3] / 1e6, 1), "automatic": round(f / pre_us / 1e6, 1)},
            "decode_M1_single_calls_weight_GBps": round(w / dec_single_us / 1e3, 1),
            "decode_M1_one_call_all7_weight_GBps": round(w / dec_all7_us / 1e3, 1),
            "per_linear": per_linear,
            "decode_M8_gate_us": round(gate_m8_us, 2),
            "merge_export_bf16": merge,
            "adamw8_adapter_step": adamw8}


def context_ceilings(torch, dev, log):
    """What the GPU does without the method: a plain device copy, and the
    library bf16 GEMM (torch.matmul, hipBLASLt) on the 70B layer's shapes at
    M = 4096 with ready bf16 weights (no 4-bit storage, no expansion).  Eager
    calls timed with HIP events on the current stream."""
    log("context ceilings: device copy, hipBLASLt bf16 GEMM")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    cu = timed(lambda: dst.copy_(src), 10)
    copy = 2 * src.numel() / cu / 1e3
    del src, dst
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    per, tot_us, tot_fl = {}, 0.0, 0
    dec_us, dec_bytes = 0.0, 0
    for name, (N, K) in L70B.items():
        X = torch.randn((M70_PRE, K), generator=g, device=dev).to(torch.bfloat16)
        Wt = (torch.randn((K, N), generator=g, device=dev) * 0.015).to(torch.bfloat16)   # [K, N], contiguous
        Y = torch.empty((M70_PRE, N), dtype=torch.bfloat16, device=dev)
        us = timed(lambda: torch.matmul(X, Wt, out=Y), 5)
        fl = 2 * M70_PRE * N * K
        per[name] = round(fl / us / 1e6, 1)
        tot_us += us
        tot_fl += fl
        X1, Y1 = X[:1].contiguous(), Y[:1].contiguous()
        dec_us += timed(lambda: torch.matmul(X1, Wt, out=Y1), 20)
        dec_bytes += 2 * N * K
        del X, Wt, Y, X1, Y1
    torch.cuda.empty_cache()
    return {"device_copy_GBps": round(copy, 1), "hipblaslt_bf16_layer_M4096_TFLOPs": round(tot_fl / tot_us / 1e6, 1),
            "hipblaslt_bf16_per_linear_TFLOPs": per,
            "dense_bf16_decode_M1_layer_us": round(dec_us, 1),
            "dense_bf16_decode_M1_weight_GBps": round(dec_bytes / dec_us / 1e3, 1),
            "note": "512 MiB device-to-device copy (read + write counted); torch.matmul on bf16 weights of the same "
                    "shapes (2MNK, no adapter, no 4-bit storage): the dense GEMM the method's expansion competes with; "
                    "dense decode: torch.matmul of one activation row by each linear's bf16 weight (1.7 GB for the "
                    "layer), the seven eager calls summed"}


def other_stages(torch, lib, dev, cap, log):
    """The rest of the path, each on its own configuration (graph-replayed)."""
    st = {}
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    randn = lambda shape, std: (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std).to(
        torch.bfloat16)

    # ---- single 4096 x 4096 projection (fp32 source weights)
    log("4096x4096 projection stages")
    N, K, R, AL = N2, K2, R2, ALPHA2
    n = N * K
    nb = n // 64
    Wf = [torch.randn((N, K), generator=g, device=dev) * 0.02 for _ in range(8)]   # 512 MiB of fp32 sources
    w0 = lib.quantize_weight(Wf[0])
    pool = [lib.NF4Weight(w0.codes.clone(), w0.absmax.clone(), w0.absmax_q.clone(), w0.scale2.clone(), N, K)
            for _ in range(64)]                                                      # 553 MB of NF4 weights
    Xd, Xp = randn((M2_DEC, K), 1.0), randn((M2_PRE, K), 1.0)
    A, B, dY = randn((R, K), 0.01), randn((N, R), 0.01), randn((M2_PRE, N), 1.0)
    deq = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    Yd = torch.empty((M2_DEC, N), dtype=torch.bfloat16, device=dev)
    Yp = torch.empty((M2_PRE, N), dtype=torch.bfloat16, device=dev)
    Hp = torch.empty((M2_PRE, R), dtype=torch.float32, device=dev)
    dX = torch.empty((M2_PRE, K), dtype=torch.bfloat16, device=dev)
    dA = torch.empty((R, K), dtype=torch.bfloat16, device=dev)
    dB = torch.empty((N, R), dtype=torch.bfloat16, device=dev)
    ws_d = lib.workspace(lib.QN_OP_FWD, M2_DEC, N, K, R, dev)
    ws_p = lib.workspace(lib.QN_OP_FWD, M2_PRE, N, K, R, dev)
    ws_b = lib.workspace(lib.QN_OP_BWD, M2_PRE, N, K, R, dev)
    wq = pool[0]
    us = {}
    us["quantize_fp32"] = graph_time_us(torch, cap, lambda: [lib.nf4_quantize(Wf[i], codes=pool[i].codes,
                                                                              absmax=pool[i].absmax)
                                                             for i in range(8)], calls=8)
    us["double_quant"] = graph_time_us(torch, cap, lambda: [lib.nf4_double_quant(pool[i].absmax,
                                                                                 absmax_q=pool[i].absmax_q,
                                                                                 scale2=pool[i].scale2)
                                                            for i in range(64)], calls=64)
    us["dequant_bf16"] = graph_time_us(torch, cap, lambda: [lib.nf4_dequant(pool[i], "bf16", out=deq)
                                                            for i in range(64)], calls=64)
    us["fwd_decode_M1"] = graph_time_us(torch, cap, lambda: [lib.qlora_linear_fwd(Xd, pool[i], A, B, AL, Y=Yd,
                                                                                  ws=ws_d)
                                                             for i in range(64)], calls=64)
    # batched decode: a few activation rows per call (the decode path runs up to M = 8)
    for mb in (2, 4, 8):
        Xm = randn((mb, K), 1.0)
        Ym = torch.empty((mb, N), dtype=torch.bfloat16, device=dev)
        wsm = lib.workspace(lib.QN_OP_FWD, mb, N, K, R, dev)
        us[f"fwd_decode_M{mb}"] = graph_time_us(torch, cap, lambda: [lib.qlora_linear_fwd(Xm, pool[i], A, B, AL,
                                                                                          Y=Ym, ws=wsm)
                                                                     for i in range(64)], calls=64)
        del Xm, Ym, wsm
    us["fwd_prefill_M2048"] = graph_time_us(torch, cap, lambda: [lib.qlora_linear_fwd(Xp, pool[i], A, B, AL, Y=Yp,
                                                                                      ws=ws_p, H=Hp)
                                                                 for i in range(8)], calls=8)
    us["bwd_M2048"] = graph_time_us(torch, cap, lambda: [lib.qlora_linear_bwd(dY, Xp, pool[i], A, B, AL,
                                                                              out=(dX, dA, dB), ws=ws_b, H=Hp)
                                                         for i in range(8)], calls=8)
    wb = nf4_bytes(N, K)
    p4 = {"us_per_call": {k: round(v, 2) for k, v in us.items()},
          "quantize_fp32_GBps": round((4 * n + n // 2 + 4 * nb) / us["quantize_fp32"] / 1e3, 1),
          "double_quant_GBps": round((5 * nb + 4 * (nb // 256)) / us["double_quant"] / 1e3, 1),
          "dequant_bf16_GBps": round((wb + 2 * n) / us["dequant_bf16"] / 1e3, 1),
          "decode_call_weight_GBps": round(wb / us["fwd_decode_M1"] / 1e3, 1),
          "prefill_call_TFLOPs": round(fwd_flops(M2_PRE, N, K, R) / us["fwd_prefill_M2048"] / 1e6, 1),
          "bwd_call_TFLOPs": round(bwd_flops(M2_PRE, N, K, R) / us["bwd_M2048"] / 1e6, 1)}
    # kernel trace of one eager pass of these calls
    # Untraced prefill calls first (about 1.5 ms of GPU work) so that the traced
    # calls enqueued meanwhile run back to back (see the 70B-layer trace).
    torch.cuda.synchronize()
    for i in range(20):
        lib.qlora_linear_fwd(Xp, pool[16 + i], A, B, AL, Y=Yp, ws=ws_p)
    lib.trace_enable(True)
    for i in range(4):
        lib.nf4_quantize(Wf[i], codes=pool[i].codes, absmax=pool[i].absmax)
        lib.nf4_double_quant(pool[i].absmax, absmax_q=pool[i].absmax_q, scale2=pool[i].scale2)
        lib.nf4_dequant(pool[i + 4], "bf16", out=deq)
        lib.qlora_linear_fwd(Xd, pool[i + 8], A, B, AL, Y=Yd, ws=ws_d)
        lib.qlora_linear_fwd(Xp, pool[i + 12], A, B, AL, Y=Yp, ws=ws_p, H=Hp)
        lib.qlora_linear_bwd(dY, Xp, pool[i + 12], A, B, AL, out=(dX, dA, dB), ws=ws_b, H=Hp)
    torch.cuda.synchronize()
    tr = lib.trace_read()
    lib.trace_enable(False)
    kern = {}
    for kind, ms in tr:
        kern.setdefault(kind, []).append(ms)
    avg = {k: sum(v) / len(v) for k, v in kern.items()}
    work = {
        "quantize": ((4 * n + n // 2 + 4 * nb), "hbm"),
        "double_quant": ((5 * nb + 4 * (nb // 256)), "hbm"),
        "dequant": ((wb + 2 * n), "hbm"),
        "gemv": ((wb + 2 * K + 2 * N + 2 * R * K), "hbm"),
        "gemm_fwd": ((2 * M2_PRE * N * K + 2 * M2_PRE * R * N), "mfma"),
        "gemm_dx": ((2 * M2_PRE * N * K + 2 * M2_PRE * R * K), "mfma"),
        # forward launch: X and A read, sH written; backward launch (H given): dY and B^T read, dH and dH^T written
        "lowrank": (((2 * M2_PRE * K + 2 * R * K + 2 * M2_PRE * R) + (2 * M2_PRE * N + 2 * R * N + 4 * M2_PRE * R)) // 2,
                    "hbm"),
        # dA = dH^T X and dB = (sH)^T dY in one launch: X, dY and the two factors read once
        "gemm_db": ((2 * M2_PRE * (K + N) + 4 * R * M2_PRE), "hbm"),
    }
    roofs = {}
    for k, (amount, bound) in work.items():
        if k not in avg:
            continue
        t = avg[k] * 1e-3
        if bound == "hbm":
            a = amount / t / 1e9
            roofs[k] = {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                        "frac": round(a / PEAK_HBM_GBPS, 4), "avg_ms": round(avg[k], 5), "work_per_launch": amount,
                        "traffic": traffic(k + "_4096", k)}
        else:
            a = amount / t / 1e12
            roofs[k] = {"bound": "mfma", "achieved": round(a, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(a / PEAK_BF16_TFLOPS, 4), "avg_ms": round(avg[k], 5), "work_per_launch": amount,
                        "traffic": traffic(k + "_4096", k)}
    p4["kernel_rooflines"] = roofs
    st["proj4096"] = p4
    del Wf, pool, w0
    torch.cuda.empty_cache()

    # ---- Qwen2.5-7B-shaped layer, forward and backward at M = 4096
    log("Qwen2.5-7B-shaped layer")
    Q = Layer(torch, lib, dev, QWEN, RQ, 0.02, [MQ], seed=7, bwd_M=MQ)
    q = {"per_linear": {}}
    for it in Q.items:
        fu = graph_time_us(torch, cap, lambda: Q.fwd(lib, MQ, [it], want_H=True))
        bu = graph_time_us(torch, cap, lambda: Q.bwd(lib, MQ, [it]))
        q["per_linear"][it["name"]] = {"fwd_us": round(fu, 1), "bwd_us": round(bu, 1),
                                       "fwd_TFLOPs": round(fwd_flops(MQ, it["N"], it["K"], RQ) / fu / 1e6, 1),
                                       "bwd_TFLOPs": round(bwd_flops(MQ, it["N"], it["K"], RQ) / bu / 1e6, 1)}
    fu = graph_time_us(torch, cap, lambda: Q.fwd(lib, MQ, want_H=True))
    bu = graph_time_us(torch, cap, lambda: Q.bwd(lib, MQ))
    qdep = Q.groups(lib, MQ, [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)])
    qall = Q.groups(lib, MQ, [tuple(QWEN)])
    gu = graph_time_us(torch, cap, lambda: [grp.run() for grp in qdep])
    au = graph_time_us(torch, cap, lambda: qall[0].run())
    q.update(fwd_single_calls_us=round(fu, 1), bwd_us=round(bu, 1),
             fwd_single_calls_TFLOPs=round(Q.flops(MQ) / fu / 1e6, 1),
             fwd_grouped_us=round(gu, 1), fwd_grouped_TFLOPs=round(Q.flops(MQ) / gu / 1e6, 1),
             fwd_one_call_all7_TFLOPs=round(Q.flops(MQ) / au / 1e6, 1),
             bwd_TFLOPs=round(Q.flops(MQ, "bwd") / bu / 1e6, 1),
             note="grouped = q,k,v | o | gate,up | down, the calls a layer's data dependencies allow")
    st["qwen2.5_7b_layer_M4096"] = q
    del Q
    torch.cuda.empty_cache()

    # ---- bulk sweep: 7.62e9 weights as 4096 x 4096 bf16 tiles, round trip
    st["bulk_round_trip_bf16_tiles"] = bulk_stage(torch, lib, dev, cap, log)

    # ---- the tiny configuration (launch-bound)
    from bit_nf4_quantized_08_amd import synth
    t = synth.tiny_inputs()
    Wt = torch.from_numpy(t["W"]).to(dev)
    wt = lib.quantize_weight(Wt)
    X, A, B, dY = (t[k].to(dev) for k in ("X", "A", "B", "dY"))
    Yt, Ht = lib.qlora_linear_fwd(X, wt, A, B, t["alpha"], want_H=True)
    M, r = X.shape[0], A.shape[0]
    gt = (torch.empty_like(X), torch.empty_like(A), torch.empty_like(B))
    wsf = lib.workspace(lib.QN_OP_FWD, M, wt.N, wt.K, r, dev)
    wsb = lib.workspace(lib.QN_OP_BWD, M, wt.N, wt.K, r, dev)

    def qdq():
        lib.nf4_quantize(Wt, codes=wt.codes, absmax=wt.absmax)
        lib.nf4_double_quant(wt.absmax, absmax_q=wt.absmax_q, scale2=wt.scale2)

    st["tiny"] = {
        "quantize_dq_us": round(graph_time_us(torch, cap, qdq, replays=50), 2),
        "fwd_us": round(graph_time_us(torch, cap, lambda: lib.qlora_linear_fwd(X, wt, A, B, t["alpha"], Y=Yt, H=Ht,
                                                                               ws=wsf), replays=50), 2),
        "bwd_us": round(graph_time_us(torch, cap, lambda: lib.qlora_linear_bwd(dY, X, wt, A, B, t["alpha"], H=Ht,
                                                                               out=gt, ws=wsb), replays=50), 2),
        "note": "launch-bound: a few microseconds of fixed cost per kernel",
    }
    return st


def bulk_stage(torch, lib, dev, cap, log):
    """The bulk quantise / double-quant / dequant round trip over 4096 x 4096
    bf16 tiles (graph-replayed): per-stage times, GB/s, round-trip error and
    stored bits per weight."""
    log("bulk round trip")
    SWEEP_WEIGHTS, TILE = 7.62e9, 4096 * 4096
    g_sw = torch.Generator(device=dev)
    g_sw.manual_seed(762)
    tiles = [(torch.randn((4096, 4096), generator=g_sw, device=dev) * 0.02).to(torch.bfloat16) for _ in range(16)]
    sw = [lib.quantize_weight(tiles[j]) for j in range(16)]
    sw_out = torch.empty((4096, 4096), dtype=torch.bfloat16, device=dev)

    def round_trip():
        # quantise with the double quantisation in the same launch, then dequantise
        for j in range(16):
            w = sw[j]
            lib.quantize_4bit(tiles[j], "nf4", codes=w.codes, absmax=w.absmax, absmax_q=w.absmax_q, scale2=w.scale2)
            lib.nf4_dequant(w, "bf16", out=sw_out)

    def round_trip_3():
        for j in range(16):
            w = sw[j]
            lib.nf4_quantize(tiles[j], codes=w.codes, absmax=w.absmax)
            lib.nf4_double_quant(w.absmax, absmax_q=w.absmax_q, scale2=w.scale2)
            lib.nf4_dequant(w, "bf16", out=sw_out)

    tile_us = graph_time_us(torch, cap, round_trip, calls=16)
    # round-trip error over the 16 tiles (bf16 source vs bf16 dequantised), on
    # the NF4 weights the round trip just wrote
    se = sr = 0.0
    for j in range(16):
        d = lib.nf4_dequant(sw[j], "bf16")
        se += float(((d.float() - tiles[j].float()).double() ** 2).sum())
        sr += float((tiles[j].double() ** 2).sum())
    tile3_us = graph_time_us(torch, cap, round_trip_3, calls=16)
    q_us = graph_time_us(torch, cap, lambda: [lib.nf4_quantize(tiles[j], codes=sw[j].codes, absmax=sw[j].absmax)
                                              for j in range(16)], calls=16)
    qdq_us = graph_time_us(torch, cap, lambda: [lib.quantize_4bit(tiles[j], "nf4", codes=sw[j].codes,
                                                                  absmax=sw[j].absmax, absmax_q=sw[j].absmax_q,
                                                                  scale2=sw[j].scale2) for j in range(16)], calls=16)
    fw = [lib.quantize_4bit(tiles[j], "fp4") for j in range(16)]      # own buffers, FP4 codes
    fq_us = graph_time_us(torch, cap, lambda: [lib.quantize_4bit(tiles[j], "fp4", codes=fw[j].codes,
                                                                 absmax=fw[j].absmax, absmax_q=fw[j].absmax_q,
                                                                 scale2=fw[j].scale2) for j in range(16)], calls=16)
    del fw
    dq_us = graph_time_us(torch, cap, lambda: [lib.nf4_double_quant(sw[j].absmax, absmax_q=sw[j].absmax_q,
                                                                    scale2=sw[j].scale2) for j in range(16)], calls=16)
    nb_t = TILE // 64
    q_bytes = 2 * TILE + TILE // 2 + 4 * nb_t
    dq_bytes = 4 * nb_t + nb_t + 4 * (nb_t // 256)
    qdq_bytes = q_bytes + nb_t + 4 * (nb_t // 256)          # quantise writes the 8-bit scales and steps too
    deq_bytes = TILE // 2 + nb_t + 4 * (nb_t // 256) + 2 * TILE
    tile_bytes = qdq_bytes + deq_bytes
    out = {
        "tile_round_trip_us": round(tile_us, 2),
        "round_trip_GBps": round(tile_bytes / tile_us / 1e3, 1),
        "tile_round_trip_3_launches_us": round(tile3_us, 2),
        "quantize_us": round(q_us, 2),
        "quantize_GBps": round(q_bytes / q_us / 1e3, 1),
        "quantize_with_double_quant_us": round(qdq_us, 2),
        "quantize_with_double_quant_GBps": round(qdq_bytes / qdq_us / 1e3, 1),
        "fp4_quantize_with_double_quant_GBps": round(qdq_bytes / fq_us / 1e3, 1),
        "double_quant_alone_us": round(dq_us, 2),
        "double_quant_alone_GBps": round(dq_bytes / dq_us / 1e3, 1),
        "sweep_7.62e9_weights_ms": round(SWEEP_WEIGHTS / TILE * tile_us * 1e-3, 2),
        "stored_bits_per_param": round((TILE // 2 + nb_t + 4 * (nb_t // 256)) * 8 / TILE, 6),
        "round_trip_rel_rmse": round((se / sr) ** 0.5, 5),
        "note": "16 distinct tiles (537 MB of bf16 source) stand in for the 454-tile stream; the round trip is "
                "qn_quantize_4bit with the double quantisation in the same launch, then nf4_dequant to bf16 "
                "(the 3-launch figure runs nf4_quantize, nf4_double_quant, nf4_dequant); sweep time = per-tile "
                "time x 7.62e9 / 4096^2",
    }
    del tiles, sw, sw_out
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
