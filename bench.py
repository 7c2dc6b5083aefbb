"""Benchmark of the NF4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--pool P]

Workload: the Llama-8B attention projection (4096 x 4096 bf16 weight ~ N(0,
0.02) with 0.1 % of entries scaled by 20; batch-1 decode with x bf16 ~ N(0,1)).
One step is one pass of the whole path over a pool of P such weights: for each
weight, nf4_quantize -> nf4_double_quant -> nf4_gemv.  The pool (P = 16 by
default, 512 MiB of bf16) is larger than the 256 MiB Infinity Cache, so every
step streams its inputs from HBM.  `value` is the algorithmic bytes of the
whole step (bf16 weights read, codes and scales written and read back, x read,
y written) divided by the step time.

Extra legs (not part of `value`): the GEMV alone over a pool of distinct
quantized weights (decode from HBM), and the dequant-into-LDS GEMM of the
QLoRA forward workload (X [4096, 4096] x NF4 W [14336, 4096] + LoRA r = 16).
`cpu_baseline` times the CPU oracle on one weight of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NF4 dequant-GEMV GB/s (% HBM peak); NF4 GEMM bf16 TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--pool", type=int, default=16)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true")
    p.add_argument("--only", choices=LEGS, default=None,
                   help="run only this extra leg (no step, no CPU baseline): for profiling one kernel family")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 64 MiB device copy kernel (for scaling HBM byte counters)")
    return p.parse_args()


# HBM bytes of the dominant kernel as read by the FETCH_SIZE / WRITE_SIZE
# counters (profiles/), kept only while the kernel's sources are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_quantize_bf16_4096x4096_traffic.json")
QUANT_SOURCES = ["k_quantize.hip", "nf4_device.h", "nf4_internal.h"]


def sources_digest(names) -> str:
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "dequant_matmul_nf4_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_digest(QUANT_SOURCES):
        return None
    return rec.get("traffic_bytes_per_launch")


def calibrate_copy():
    """A plain elementwise copy (y = -x) of 64 MiB of float32: the kernel reads
    and writes exactly 64 MiB, which fixes the scale of the byte counters."""
    import torch
    n = 16 << 20
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "neg_copy", "bytes_read": 4 * n, "bytes_written": 4 * n, "launches": 5}))
    return 0


def step_bytes(rows: int, cols: int, m: int = 1) -> dict:
    """Algorithmic bytes of quantize, double quant and GEMV for one weight."""
    n = rows * cols
    nb = n // 64
    ng = -(-nb // 256)
    quant = 2 * n + n // 2 + 4 * nb
    dq = 4 * nb + nb + 4 * ng + 4
    gemv = n // 2 + nb + 4 * ng + 4 + 2 * m * cols + 2 * m * rows
    return {"quantize": quant, "double_quant": dq, "gemv": gemv}


def capture_graph(torch, fn):
    """Captures the launches fn() makes on the current stream into a HIP graph."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        fn()
    return g


class EventTimer:
    """HIP events recorded on the stream the kernels run on."""

    def __init__(self, torch, stream):
        self.torch, self.stream, self.pairs = torch, stream, []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e

    def stop(self, s):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs.append((s, e))

    def mean_us(self):
        return 1e3 * sum(a.elapsed_time(b) for a, b in self.pairs) / max(1, len(self.pairs))

    def median_us(self):
        v = sorted(1e3 * a.elapsed_time(b) for a, b in self.pairs)
        return v[len(v) // 2] if v else 0.0


def only_leg(name: str) -> int:
    import torch

    import dequant_matmul_nf4_amd as nf4
    import synthetic as syn

    nf4.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    res = extra_legs(torch, nf4, syn, dev, torch.cuda.current_stream(), EventTimer, only=name)
    print(json.dumps({"leg": name, **res}), flush=True)
    return 0


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; use --gpus 1"}))
        print("bench.py: only --gpus 1 is supported (single-GPU build)", file=sys.stderr)
        return 2

    if args.calibrate_copy:
        return calibrate_copy()
    if args.only:
        return only_leg(args.only)

    import numpy as np
    import torch

    import dequant_matmul_nf4_amd as nf4
    import synthetic as syn

    nf4.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    rows = cols = 4096
    P = args.pool

    print(f"[bench] generating {P} weights 4096x4096 bf16", file=sys.stderr, flush=True)
    ws = [syn.c2_weight(pool_index=i).to(dev) for i in range(P)]
    x = syn.c2_inputs()["x"].to(dev)
    n = rows * cols
    nb = n // 64
    bufs = []
    for _ in range(P):
        bufs.append(dict(
            packed=torch.empty(n // 2, dtype=torch.uint8, device=dev),
            absmax=torch.empty(nb, dtype=torch.float32, device=dev),
            q=torch.empty(nb, dtype=torch.int8, device=dev),
            s2=torch.empty(-(-nb // 256), dtype=torch.float32, device=dev),
            mean=torch.empty(1, dtype=torch.float32, device=dev),
            y=torch.empty((1, rows), dtype=torch.bfloat16, device=dev),
        ))
    dq_ws = torch.empty(nf4.nf4_double_quant_workspace(nb), dtype=torch.uint8, device=dev)
    Wq = [nf4.NF4Weight(b["packed"], rows, cols, qabsmax=b["q"], absmax2=b["s2"], mean=b["mean"]) for b in bufs]

    def run_quantize():
        for i in range(P):
            nf4.nf4_quantize(ws[i], bufs[i]["packed"], bufs[i]["absmax"])

    def run_double_quant():
        for b in bufs:
            nf4.nf4_double_quant(b["absmax"], b["q"], b["s2"], b["mean"], dq_ws)

    def run_gemv():
        for i in range(P):
            nf4.nf4_gemv(Wq[i], x, bufs[i]["y"])

    # One step = quantize every weight of the pool, double-quantize every
    # absmax, then the decode GEMV on every weight: three HIP graphs replayed
    # back to back on the current stream, with events between them (so the
    # per-kernel averages come from the timed region itself).
    print("[bench] eager warmup and graph capture", file=sys.stderr, flush=True)
    for f in (run_quantize, run_double_quant, run_gemv):
        f()
    torch.cuda.synchronize()
    graphs = [capture_graph(torch, f) for f in (run_quantize, run_double_quant, run_gemv)]
    torch.cuda.synchronize()

    def one_step(ev=None):
        for j, g in enumerate(graphs):
            if ev is not None:
                ev[j].record(stream)
            g.replay()
        if ev is not None:
            ev[3].record(stream)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_step(evs[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    sb = step_bytes(rows, cols)
    bytes_per_step = P * sum(sb.values())
    value = bytes_per_step * args.steps / elapsed / 1e9
    phase_us = [1e3 * sum(e[j].elapsed_time(e[j + 1]) for e in evs) / (args.steps * P) for j in range(3)]
    q_us, d_us, g_us = phase_us
    q_gbs = sb["quantize"] / (q_us * 1e-6) / 1e9
    g_gbs_hot = sb["gemv"] / (g_us * 1e-6) / 1e9

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "Llama-8B attention projection 4096x4096 bf16, N(0,0.02) + 0.1% outliers x20; "
                        "NF4 blocksize 64 + double quant (int8, groups of 256); batch-1 decode GEMV",
            "pool_weights": P,
            "step": "nf4_quantize of every pool weight, nf4_double_quant of every absmax, nf4_gemv on every "
                    "weight (three HIP graphs)",
            "bytes_per_step": bytes_per_step,
        },
        "roofline": {
            "kernel": "k_quantize<bf16>",
            "bound": "hbm",
            "achieved": round(q_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(q_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "bytes_per_launch": sb["quantize"],
            "avg_launch_us": round(q_us, 3),
        },
        "kernels_in_step": {
            "quantize_us": round(q_us, 3),
            "double_quant_us": round(d_us, 3),
            "gemv_us": round(g_us, 3),
            "gemv_GBps_packed_just_written": round(g_gbs_hot, 1),
        },
    }

    if not args.no_extra:
        out.update(extra_legs(torch, nf4, syn, dev, stream, EventTimer))

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(np, syn)

    out["host"] = {"cpu": platform.processor() or platform.machine(), "gpu": torch.cuda.get_device_name(dev),
                   "hip": torch.version.hip}
    print(json.dumps(out), flush=True)
    return 0


LEGS = ("hbm", "gemv-decode", "gemv-mlp", "gemv-70b", "stack-70b", "gemm", "qlora-backward", "lora-merge")


def extra_legs(torch, nf4, syn, dev, stream, EventTimer, only=None):
    """GEMV alone from HBM (decode), the Llama-8B MLP and 70B-layer GEMVs, and
    the QLoRA forward GEMM; `only` runs a single one of LEGS."""
    res = {}
    g = torch.Generator(device=dev)
    if only in (None, "hbm"):
        res.update(leg_hbm_calibration(torch, dev, stream, EventTimer))
    if only in (None, "gemv-decode"):
        res.update(leg_gemv_decode(torch, nf4, syn, dev, stream, EventTimer, g))
    if only in (None, "gemv-mlp", "gemv-70b"):
        res.update(legs_gemv_pools(torch, nf4, dev, stream, EventTimer, g, only))
    if only in (None, "stack-70b"):
        res.update(leg_stack_70b(torch, nf4, syn, dev, stream, EventTimer))
    if only in (None, "gemm"):
        res.update(leg_gemm(torch, nf4, dev, stream, EventTimer, g))
    if only in (None, "qlora-backward"):
        res.update(leg_qlora_backward(torch, nf4, dev, stream, EventTimer, g))
    if only in (None, "lora-merge"):
        res.update(leg_lora_merge(torch, nf4, dev, stream, EventTimer, g))
    return res


def _median_call(torch, stream, EventTimer, fn, reps=30, warm=5):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    t = EventTimer(torch, stream)
    for _ in range(reps):
        s = t.start()
        fn()
        t.stop(s)
    torch.cuda.synchronize()
    return t.median_us()


def leg_qlora_backward(torch, nf4, dev, stream, EventTimer, g):
    """The backward of the QLoRA forward GEMM (X 4096x4096, NF4(DQ) W
    14336x4096, LoRA r = 16, alpha = 32): the input gradient through the
    frozen base, dX = dY.deq(W) + s.(dY.B).A, and the adapter gradients dA,
    dB (medians of 30 calls)."""
    print("[bench] qlora backward leg", file=sys.stderr, flush=True)
    M, N, K, r = 4096, 14336, 4096, 16
    s_l = 32.0 / r
    g.manual_seed(4_005)
    X = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
    g.manual_seed(4_000)
    W = nf4.quantize_weight((torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16),
                            double_quant=True)
    g.manual_seed(4_006)
    A = (torch.randn((r, K), generator=g, device=dev) * 0.01).to(torch.bfloat16)
    g.manual_seed(4_007)
    B = (torch.randn((N, r), generator=g, device=dev) * 0.01).to(torch.bfloat16)
    g.manual_seed(4_008)
    dY = torch.randn((M, N), generator=g, device=dev).to(torch.bfloat16)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dA = torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = torch.empty((N, r), dtype=torch.float32, device=dev)
    ws_dx = torch.empty(max(nf4.nf4_gemm_dx_workspace(M, N, r), 1), dtype=torch.uint8, device=dev)
    ws_g = torch.empty(max(nf4.nf4_lora_grads_workspace(M, N, K, r), 1), dtype=torch.uint8, device=dev)
    us_dx = _median_call(torch, stream, EventTimer, lambda: nf4.nf4_gemm_dx(W, dY, dX, A, B, s_l, ws_dx))
    us_g = _median_call(torch, stream, EventTimer,
                        lambda: nf4.nf4_lora_grads(X, dY, A, B, s_l, da=dA, db=dB, workspace=ws_g))
    fl_dx = 2.0 * M * N * K + 2.0 * M * N * r + 2.0 * M * r * K
    tf = fl_dx / (us_dx * 1e-6) / 1e12
    Wd = nf4.nf4_dequantize(W, out_dtype=torch.bfloat16)
    us_lib = _median_call(torch, stream, EventTimer, lambda: torch.matmul(dY, Wd))
    del Wd
    return {"qlora_backward": {
        "workload": "dY 4096x14336 bf16, NF4(DQ) W 14336x4096, LoRA r=16 alpha=32: dX, dA, dB",
        "gemm_dx_us": round(us_dx, 1),
        "gemm_dx_TFLOPs": round(tf, 1),
        "gemm_dx_frac_mfma_bf16_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "lora_grads_us": round(us_g, 1),
        "timing": "medians of 30 calls after 5 warm-ups (dX call includes its LoRA prep; grads include both thin products)",
        "calibration_torch_matmul_bf16": {
            "what": "torch.matmul (hipBLASLt) dY . W on the dequantized bf16 weight, no LoRA",
            "us": round(us_lib, 1),
            "TFLOPs": round(2.0 * M * N * K / (us_lib * 1e-6) / 1e12, 1),
        },
    }}


FP64_VECTOR_PEAK_TFLOPS = 78.6


def leg_lora_merge(torch, nf4, dev, stream, EventTimer, g):
    """The LoRA merge on the QLoRA shape: W 14336x4096 (NF4 + double quant),
    r = 16, alpha = 32, merged into a dense bf16 copy (median of 20)."""
    print("[bench] lora merge leg", file=sys.stderr, flush=True)
    N, K, r = 14336, 4096, 16
    g.manual_seed(4_000)
    W = nf4.quantize_weight((torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16),
                            double_quant=True)
    g.manual_seed(4_006)
    A = (torch.randn((r, K), generator=g, device=dev) * 0.01).to(torch.bfloat16)
    g.manual_seed(4_007)
    B = (torch.randn((N, r), generator=g, device=dev) * 0.01).to(torch.bfloat16)
    out = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        nf4.nf4_lora_merge(W, A, B, 2.0, out=out)
    torch.cuda.synchronize()
    t = EventTimer(torch, stream)
    for _ in range(20):
        s = t.start()
        nf4.nf4_lora_merge(W, A, B, 2.0, out=out)
        t.stop(s)
    torch.cuda.synchronize()
    us = t.median_us()
    sb = step_bytes(N, K)
    nbytes = sb["gemv"] - 2 * K - 2 * N + 2 * N * K + 2 * r * (N + K)  # NF4 + scales in, bf16 out, adapters
    flops = 2.0 * r * N * K
    del W, out
    return {"lora_merge": {
        "workload": "W 14336x4096 NF4+DQ + s.B.A (r=16, s=2) -> dense bf16, float64 rank-16 sums",
        "us": round(us, 1),
        "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
        "frac_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "fp64_TFLOPs": round(flops / (us * 1e-6) / 1e12, 2),
        "frac_fp64_vector_peak": round(flops / (us * 1e-6) / 1e12 / FP64_VECTOR_PEAK_TFLOPS, 4),
    }}


def leg_stack_70b(torch, nf4, syn, dev, stream, EventTimer, layers=80, gemv_passes=20):
    """The 80-layer 70B-shaped stack.  Layer by layer, the seven bf16 weights
    (q, k, v, o, gate, up, down) are drawn on the device (untimed) and then
    quantized and double-quantized into a persistent NF4 store (timed: one HIP
    graph of the 7 x 3 launches per layer).  Afterwards the decode GEMV runs
    over one layer's seven matrices, a different stored layer on every pass,
    so that no pass finds its 441 MB in the last-level cache."""
    print(f"[bench] 70B stack leg: {layers} layers", file=sys.stderr, flush=True)
    LAYER_70B = [syn.C5_SHAPES[name] for name in syn.C5_ORDER]
    g = torch.Generator(device=dev)
    src = [torch.empty(sh, dtype=torch.bfloat16, device=dev) for sh in LAYER_70B]
    nbs = [r * c // 64 for r, c in LAYER_70B]
    absmax = [torch.empty(nb, dtype=torch.float32, device=dev) for nb in nbs]
    dq_ws = torch.empty(nf4.nf4_double_quant_workspace(max(nbs)), dtype=torch.uint8, device=dev)
    store, t = [], EventTimer(torch, stream)
    for layer in range(layers):
        Ws = []
        for (r, c), nb in zip(LAYER_70B, nbs):
            Ws.append(nf4.NF4Weight(torch.empty(r * c // 2, dtype=torch.uint8, device=dev), r, c,
                                    qabsmax=torch.empty(nb, dtype=torch.int8, device=dev),
                                    absmax2=torch.empty(-(-nb // 256), dtype=torch.float32, device=dev),
                                    mean=torch.empty(1, dtype=torch.float32, device=dev)))

        def run():
            for w, W, am in zip(src, Ws, absmax):
                nf4.nf4_quantize(w, W.packed, am)
                nf4.nf4_double_quant(am, W.qabsmax, W.absmax2, W.mean, dq_ws)

        graph = capture_graph(torch, run)
        graph.replay()  # first launch of the graph (upload), on the previous layer's data; untimed
        for j, name in enumerate(syn.C5_ORDER):
            src[j].copy_(syn.c5_weight_device(layer, name, device=dev))
        s = t.start()
        graph.replay()
        t.stop(s)
        torch.cuda.synchronize()
        del graph
        store.append(Ws)
    q_us = [1e3 * a.elapsed_time(b) for a, b in t.pairs]
    n_layer = sum(r * c for r, c in LAYER_70B)
    alg_layer = sum(step_bytes(r, c)["quantize"] + step_bytes(r, c)["double_quant"] for r, c in LAYER_70B)
    total_s = sum(q_us) * 1e-6
    del src, absmax

    g.manual_seed(5_000_009)
    xs = {c: (torch.randn((1, c), generator=g, device=dev)).to(torch.bfloat16) for _, c in LAYER_70B}
    ys = [torch.empty((1, r), dtype=torch.bfloat16, device=dev) for r, _ in LAYER_70B]
    step = max(1, layers // gemv_passes)
    pass_layers = [(i * step) % layers for i in range(gemv_passes)]
    graphs = []
    for layer in pass_layers:
        def run_gemv(Ws=store[layer]):
            for W, yy in zip(Ws, ys):
                nf4.nf4_gemv(W, xs[W.cols], yy)
        run_gemv()
        graphs.append(capture_graph(torch, run_gemv))
    torch.cuda.synchronize()
    tg = EventTimer(torch, stream)
    for gr in graphs:
        s = tg.start()
        gr.replay()
        tg.stop(s)
    torch.cuda.synchronize()
    g_us = sorted(1e3 * a.elapsed_time(b) for a, b in tg.pairs)
    g_med = g_us[len(g_us) // 2]
    g_bytes = sum(step_bytes(r, c)["gemv"] for r, c in LAYER_70B)
    del graphs, store
    return {"stack_70b": {
        "workload": f"{layers} layers of q,o 8192x8192, k,v 1024x8192, gate,up 28672x8192, down 8192x28672, bf16 "
                    "N(0,0.02) drawn per layer on the device; NF4 + double quant into a persistent store",
        "layers": layers,
        "quantize_dq_us_per_layer": round(sum(q_us) / layers, 1),
        "quantize_dq_input_GBps": round(2 * n_layer * layers / total_s / 1e9, 1),
        "quantize_dq_algorithmic_GBps": round(alg_layer * layers / total_s / 1e9, 1),
        "quantize_dq_frac_hbm_peak": round(alg_layer * layers / total_s / 1e9 / HBM_PEAK_GBS, 4),
        "nf4_store_GB": round(layers * g_bytes / 1e9, 2),
        "gemv_layer_rotating": {
            "passes": gemv_passes, "median_us": round(g_med, 2),
            "GBps": round(g_bytes / (g_med * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(g_bytes / (g_med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        },
    }}


def leg_hbm_calibration(torch, dev, stream, EventTimer):
    """What the memory system gives vendor kernels on this GPU, as the
    measured-achievable context for the HBM-bound kernels: torch's device copy
    (read + write) and a full reduction (read only) over 2 GiB."""
    print("[bench] HBM calibration", file=sys.stderr, flush=True)
    n = 1 << 30  # bf16 elements: 2 GiB
    a = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    out = {}
    for what, fn, nbytes in (("copy", lambda: b.copy_(a), 4 * n), ("sum", lambda: a.sum(dtype=torch.float32), 2 * n)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t = EventTimer(torch, stream)
        for _ in range(10):
            s = t.start()
            fn()
            t.stop(s)
        torch.cuda.synchronize()
        us = t.median_us()
        out[what] = {"GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "us": round(us, 1)}
    del a, b
    return {"hbm_calibration": {"what": "torch copy_ (2 GiB read + 2 GiB write) and sum (2 GiB read), median of 10",
                                **out}}


def leg_gemv_decode(torch, nf4, syn, dev, stream, EventTimer, g):
    res = {}
    rows = cols = 4096
    print("[bench] gemv-only leg", file=sys.stderr, flush=True)
    pool = 64
    Ws = []
    for i in range(pool):
        g.manual_seed(7_000 + i)
        w = (torch.randn((rows, cols), generator=g, device=dev) * 0.02).to(torch.bfloat16)
        Ws.append(nf4.quantize_weight(w, double_quant=True))
        del w
    x = syn.c2_inputs()["x"].to(dev)
    y = torch.empty((1, rows), dtype=torch.bfloat16, device=dev)

    def run():
        for W in Ws:
            nf4.nf4_gemv(W, x, y)

    run()
    torch.cuda.synchronize()
    graph = capture_graph(torch, run)
    graph.replay()
    torch.cuda.synchronize()
    t = EventTimer(torch, stream)
    s = t.start()
    reps = 20
    for _ in range(reps):
        graph.replay()
    t.stop(s)
    torch.cuda.synchronize()
    per_call_us = t.mean_us() / (reps * pool)
    gb = step_bytes(rows, cols)["gemv"]
    res["gemv_decode_hbm"] = {
        "workload": "4096x4096 NF4+DQ, M=1, pool of 64 distinct weights (557 MB)",
        "per_call_us": round(per_call_us, 3),
        "GBps": round(gb / (per_call_us * 1e-6) / 1e9, 1),
        "frac_hbm_peak": round(gb / (per_call_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
    }
    del Ws
    return res


def legs_gemv_pools(torch, nf4, dev, stream, EventTimer, g, only=None):
    """Larger decode GEMVs: the Llama-8B MLP (M = 1, 4, 16) and one 70B-shaped layer."""
    res = {}

    def gemv_pool(shapes, reps, label, m=1, dq_type="int8"):
        Wl = []
        for i, (r_, c_) in enumerate(shapes):
            g.manual_seed(9_000 + i)
            w = (torch.randn((r_, c_), generator=g, device=dev) * 0.02).to(torch.bfloat16)
            Wl.append(nf4.quantize_weight(w, double_quant=True, dq_type=dq_type))
            del w
        xs = {c_: (torch.randn((m, c_), generator=g, device=dev)).to(torch.bfloat16) for _, c_ in shapes}
        ys = [torch.empty((m, r_), dtype=torch.bfloat16, device=dev) for r_, _ in shapes]

        def run():
            for W, yy in zip(Wl, ys):
                nf4.nf4_gemv(W, xs[W.cols], yy)

        run()
        torch.cuda.synchronize()
        graph = capture_graph(torch, run)
        graph.replay()
        torch.cuda.synchronize()
        t = EventTimer(torch, stream)
        s = t.start()
        for _ in range(reps):
            graph.replay()
        t.stop(s)
        torch.cuda.synchronize()
        total_us = t.mean_us() / reps
        nbytes = sum(step_bytes(r_, c_, m)["gemv"] for r_, c_ in shapes)
        del Wl
        return {"workload": label, "m": m, "us_per_pass": round(total_us, 2),
                "GBps": round(nbytes / (total_us * 1e-6) / 1e9, 1),
                "frac_hbm_peak": round(nbytes / (total_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}

    print("[bench] gemv MLP / 70B-layer legs", file=sys.stderr, flush=True)
    if only in (None, "gemv-mlp"):
        mlp = [(14336, 4096), (14336, 4096), (4096, 14336)] * 6
        label = ("Llama-8B MLP gate/up 14336x4096 + down 4096x14336, NF4+DQ, 6 distinct triples (545 MB) per pass")
        res["gemv_mlp_8b"] = gemv_pool(mlp, 10, label + ", M=1")
        res["gemv_mlp_8b_m4"] = gemv_pool(mlp, 10, label + ", M=4", m=4)
        res["gemv_mlp_8b_m16"] = gemv_pool(mlp, 10, label + ", M=16", m=16)
    if only in (None, "gemv-70b"):
        layer = [(8192, 8192), (1024, 8192), (1024, 8192), (8192, 8192), (28672, 8192), (28672, 8192),
                 (8192, 28672)]
        res["gemv_layer_70b"] = gemv_pool(layer, 10, "70B-shaped layer q,k,v,o,gate,up,down NF4+DQ, M=1 (442 MB)")
        res["gemv_layer_70b_fp8_scales"] = gemv_pool(
            layer, 10, "the same layer with float8 (E4M3) second-level scales, M=1", dq_type="fp8")
        res["double_quant_70b_gate"] = leg_dq_kinds(torch, nf4, dev, stream, EventTimer, g)
    return res


def leg_dq_kinds(torch, nf4, dev, stream, EventTimer, g):
    """Double quantization of the 3.67 M scales of one 28672x8192 weight with
    the int8 and the float8 second level (medians of 20 calls)."""
    g.manual_seed(9_100)
    w = (torch.randn((28672, 8192), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    _, absmax = nf4.nf4_quantize(w)
    del w
    nb = absmax.numel()
    out = {}
    for kind in ("int8", "fp8"):
        q, s2, mean = nf4.nf4_double_quant(absmax, fp8=kind == "fp8")
        ws = torch.empty(nf4.nf4_double_quant_workspace(nb), dtype=torch.uint8, device=dev)
        us = _median_call(torch, stream, EventTimer,
                          lambda: nf4.nf4_double_quant(absmax, q, s2, mean, ws, fp8=kind == "fp8"), reps=20)
        out[kind] = {"us": round(us, 2), "GBps_algorithmic": round(nb * 5.016 / (us * 1e-6) / 1e9, 1)}
    return {"workload": "scales of one 28672x8192 NF4 weight (3.67 M)", **out}


def leg_gemm(torch, nf4, dev, stream, EventTimer, g):
    res = {}
    print("[bench] gemm leg", file=sys.stderr, flush=True)
    M, N, K, r = 4096, 14336, 4096, 16
    g.manual_seed(4_005)
    X = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
    g.manual_seed(4_000)
    W = nf4.quantize_weight((torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16),
                            double_quant=True)
    g.manual_seed(4_006)
    A = (torch.randn((r, K), generator=g, device=dev) * 0.01).to(torch.bfloat16)
    g.manual_seed(4_007)
    B = (torch.randn((N, r), generator=g, device=dev) * 0.01).to(torch.bfloat16)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    wsb = torch.empty(nf4.nf4_gemm_workspace(M, N, r), dtype=torch.uint8, device=dev)
    # median of 50 event-timed calls after 10 warm-ups
    for _ in range(10):
        nf4.nf4_gemm(W, X, Y, A, B, 2.0, wsb)
    torch.cuda.synchronize()
    t = EventTimer(torch, stream)
    reps = 50
    for _ in range(reps):
        s = t.start()
        nf4.nf4_gemm(W, X, Y, A, B, 2.0, wsb)
        t.stop(s)
    torch.cuda.synchronize()
    us = t.median_us()
    flops = 2.0 * M * N * K + 2.0 * M * K * r + 2.0 * M * r * N
    tf = flops / (us * 1e-6) / 1e12
    res["gemm_qlora_forward"] = {
        "workload": "X 4096x4096 bf16 . NF4(DQ) W 14336x4096^T + LoRA r=16 alpha=32",
        "us": round(us, 1),
        "us_mean": round(t.mean_us(), 1),
        "TFLOPs": round(tf, 1),
        "frac_mfma_bf16_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "timing": f"median of {reps} calls (LoRA prep + GEMM) after 10 warm-ups",
    }
    # Calibration only (not part of the path): the vendor library's plain bf16
    # GEMM of the same shape on an already dequantized weight, no LoRA.
    Wd = nf4.nf4_dequantize(W, out_dtype=torch.bfloat16)
    for _ in range(10):
        torch.nn.functional.linear(X, Wd)
    torch.cuda.synchronize()
    t = EventTimer(torch, stream)
    for _ in range(reps):
        s = t.start()
        torch.nn.functional.linear(X, Wd)
        t.stop(s)
    torch.cuda.synchronize()
    us_lib = t.median_us()
    res["gemm_qlora_forward"]["calibration_torch_linear_bf16"] = {
        "what": "torch.nn.functional.linear (hipBLASLt) on the dequantized bf16 weight, same M, N, K, no LoRA",
        "us": round(us_lib, 1),
        "TFLOPs": round(2.0 * M * N * K / (us_lib * 1e-6) / 1e12, 1),
    }
    del Wd
    return res


def cpu_baseline(np, syn, min_seconds: float = 10.0):
    """The CPU oracle (as it stands) on one weight of the same workload:
    quantize, double quant, dequantize and the float64 GEMV, single-threaded,
    repeated until at least `min_seconds` have passed."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
    rows = cols = 4096
    w = syn.bf16_to_f32(syn.c2_weight()).reshape(-1)
    x = syn.bf16_to_f32(syn.c2_inputs()["x"])
    import contextlib
    ctx = threadpool_limits(1) if threadpool_limits else contextlib.nullcontext()
    reps = 0
    with ctx:
        t0 = time.perf_counter()
        while True:
            p, a = oracle.quantize(w)
            q, s2, mu = oracle.double_quant(a)
            wdeq = oracle.bf16_bits_to_f32(oracle.dequantize(p, w.size, qabsmax=q, absmax2=s2, mean=mu, out="bf16"))
            oracle.matmul_ref(x, wdeq.reshape(rows, cols))
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    sb = step_bytes(rows, cols)
    return {
        "value": round(reps * sum(sb.values()) / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{reps} passes over one 4096x4096 weight of the workload: quantize + double quant + "
                  "dequant + float64 GEMV",
        "seconds": round(dt, 2),
    }


if __name__ == "__main__":
    sys.exit(main())
