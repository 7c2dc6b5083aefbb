"""Benchmark of the NF4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L]

Workload: the largest configuration, a 70B-shaped layer stack of L = 80
layers (q, o 8192 x 8192; k, v 1024 x 8192; gate, up 28672 x 8192; down
8192 x 28672; bf16 ~ N(0, 0.02) drawn on the device layer by layer), each
weight quantized to NF4 with int8 double quantization into a persistent
store (35.3 GB; the stack's quantize + double-quant throughput is reported
beside the headline).  One step is the decode GEMV (m = 1) over the seven
matrices of one stored layer; consecutive steps take different layers, so a
step never finds its 442 MB in the 256 MB last-level cache.  `value` is the
algorithmic bytes of the steps (NF4 codes, int8 scale codes, group scales,
the mean, x and y) divided by their wall time.

Extra legs (not part of `value`): the memory-system calibration (torch copy
and sum, and a plain streaming-read kernel of our own), the 1024^2 round trip
(microseconds), the 4096^2 quantize + double quant + GEMV composite and the
GEMV alone over a pool of 4096^2 weights, the Llama-8B MLP GEMVs at m = 1, 4,
16, the dequantize-and-multiply matrix-core GEMM of the QLoRA forward
(X [4096, 4096] x NF4 W [14336, 4096] + LoRA r = 16, the GEMM roofline), its
backward, the LoRA merge, and the double quantization with both second-level
types.  `--only layer-forms` compares the layer's decode GEMV as seven
launches, four batched launches and one batched launch.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
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
WARM_SECONDS = 0.2
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--layers", type=int, default=80, help="layers of the 70B-shaped stack (at most 80)")
    p.add_argument("--pool", type=int, default=16, help="weights in the pool of the 4096x4096 step leg")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true")
    p.add_argument("--only", choices=LEGS, default=None,
                   help="run only this extra leg (no step, no CPU baseline): for profiling one kernel family")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 64 MiB device copy kernel (for scaling HBM byte counters)")
    return p.parse_args()


# HBM bytes of the dominant kernel as read by the FETCH_SIZE / WRITE_SIZE
# counters (profiles/), kept only while the kernel's sources are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_gemv_batch_70b_layer_traffic.json")
GEMV_SOURCES = ["k_gemv_batch.hip", "gemv_rows.h", "nf4_device.h", "nf4_internal.h"]


def sources_digest(names) -> str:
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "dequant_matmul_nf4_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


GEMM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_gemm_qlora_forward_traffic.json")
GEMM_SOURCES = ["k_gemm.hip", "gemm_tiles.h", "nf4_device.h", "nf4_internal.h"]


def measured_traffic(path=TRAFFIC_FILE, sources=GEMV_SOURCES):
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_digest(sources):
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


def host_info(torch, dev) -> dict:
    """The machine the numbers come from: CPU model, the cores this process
    may run on, the BLAS threads numpy uses, the GPU and the HIP version."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = sum(int(i.get("num_threads", 0)) for i in threadpool_info() if i.get("user_api") == "blas") or None
    except Exception:  # pragma: no cover
        pass
    return {"cpu": model, "cores_allowed": len(os.sched_getaffinity(0)), "blas_threads": blas,
            "gpu": torch.cuda.get_device_name(dev), "hip": torch.version.hip}


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

    # The 70B-shaped stack, quantized and double-quantized into a persistent
    # NF4 store layer by layer (timed as the stack's own figure).
    store, stack = build_stack_70b(torch, nf4, syn, dev, stream, EventTimer, args.layers)
    shapes = [syn.C5_SHAPES[name] for name in syn.C5_ORDER]
    step_bytes_layer = sum(step_bytes(r, c)["gemv"] for r, c in shapes)

    # One step: the decode GEMV (m = 1) over the seven matrices of one stored
    # layer in one nf4_gemv_batched call (one launch), each matrix with its
    # layer input (q, k, v: the attention input; o: the attention output;
    # gate, up: the MLP input; down: the MLP hidden state).  Consecutive steps
    # take layers 37 apart, so no step finds its 442 MB in the 256 MB
    # last-level cache.  The warmup steps and the timed steps are one HIP
    # graph each (W and K launches back to back), so the timed region holds
    # the K launches and no host dispatch gap; HIP events on the stream the
    # graph runs on bracket it.  The decode-order form (four launches: o and
    # down wait for the results before them in a real model) and seven single
    # launches are measured beside it.
    xs = layer_inputs(torch, dev)
    ys = [torch.empty((1, r), dtype=torch.bfloat16, device=dev) for r, _ in shapes]
    L = len(store)
    order = [(37 * k) % L for k in range(max(args.steps, args.warmup))]
    print(f"[bench] capturing {args.warmup} warmup and {args.steps} timed steps over {L} stored layers",
          file=sys.stderr, flush=True)
    warm = capture_layer_steps(torch, nf4, store, order[:args.warmup], xs, ys, "one")
    timed = capture_layer_steps(torch, nf4, store, order[:args.steps], xs, ys, "one")
    torch.cuda.synchronize()

    # The W warm-up steps are replayed until at least WARM_SECONDS have passed:
    # under sustained streaming the GPU's clock first dips (a power transient
    # of a few milliseconds, 10-15% slower launches) and then settles, and the
    # timed steps should see the settled state, not the transient.
    print("[bench] warmup", file=sys.stderr, flush=True)
    t_w = time.perf_counter()
    warm_passes = 0
    while warm_passes == 0 or time.perf_counter() - t_w < WARM_SECONDS:
        warm.replay()
        warm_passes += 1
        torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    timed.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    mean_us = 1e3 * ev0.elapsed_time(ev1) / args.steps
    value = step_bytes_layer * args.steps / elapsed / 1e9
    achieved = step_bytes_layer / (mean_us * 1e-6) / 1e9
    del warm, timed
    read_gbs = None

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
        "dtype": "nf4-weights bf16-x f32-accumulate",
        "data": "synthetic",
        "config": {
            "workload": f"70B-shaped layer stack, {L} layers of q,o 8192x8192, k,v 1024x8192, gate,up 28672x8192, "
                        "down 8192x28672 (bf16 N(0,0.02) drawn on the device), NF4 blocksize 64 + int8 double quant "
                        "(groups of 256) in a persistent store; decode GEMV y = x.deq(W)^T at m=1 over the seven "
                        "matrices of one stored layer per step, a different layer each step",
            "layers": L,
            "step": "one nf4_gemv_batched call (one launch) over q, k, v, o, gate, up, down of one stored layer, "
                    "each with its layer input (attention input for q, k, v; attention output for o; MLP input for "
                    "gate, up; MLP hidden state for down); the K timed steps are one HIP graph of K launches",
            "bytes_per_step": step_bytes_layer,
            "warmup_note": f"the {args.warmup} warm-up steps (one graph) replayed {warm_passes} times, "
                           f"at least {WARM_SECONDS} s, before the timed steps",
            "bytes_per_weight": "0.5 codes + 1/64 int8 scale codes + 4/16384 group scales; plus x and y",
        },
        "roofline": {
            "kernel": "k_gemv_batch (one launch per step)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "bytes_per_launch": step_bytes_layer,
            "avg_launch_us": round(mean_us, 3),
            "timing": "HIP events on the graph's stream around the K timed launches, divided by K",
        },
    }
    out["stack_70b"] = stack

    if not args.no_extra:
        extra = extra_legs(torch, nf4, syn, dev, stream, EventTimer)
        read_gbs = extra.get("hbm_calibration", {}).get("stream_read", {}).get("GBps")
        gemm = extra.get("gemm_qlora_forward")
        if gemm:
            out["roofline_gemm"] = {
                "kernel": "k_gemm (QLoRA forward call: LoRA prep + k_gemm)",
                "bound": "mfma",
                "achieved": gemm["TFLOPs"],
                "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s",
                "frac": round(gemm["TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(GEMM_TRAFFIC_FILE, GEMM_SOURCES),
                "flops_per_launch": gemm["flops"],
                "avg_launch_us": gemm["us_mean"],
            }
            cal = gemm.get("calibration_torch_linear_bf16", {}).get("TFLOPs")
            if cal:
                # the vendor library's plain bf16 GEMM of the same shape: the
                # measured-achievable matrix-core rate of this GPU here
                out["roofline_gemm"]["measured_bf16_gemm_TFLOPs"] = cal
                out["roofline_gemm"]["frac_of_measured_bf16_gemm"] = round(gemm["TFLOPs"] / cal, 4)
        out.update(extra)
    if read_gbs:
        out["roofline"]["measured_read_GBps"] = read_gbs
        out["roofline"]["frac_of_measured_read"] = round(achieved / read_gbs, 4)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(np, syn, torch, dev)

    out["host"] = host_info(torch, dev)
    del store
    print(json.dumps(out), flush=True)
    return 0


def layer_inputs(torch, dev):
    """The decode inputs of a 70B-shaped layer (bf16 ~ N(0, 1)): the
    attention input (q, k, v), the attention output (o), the MLP input
    (gate, up) and the MLP hidden state (down)."""
    g = torch.Generator(device=dev)
    g.manual_seed(5_000_009)
    return {name: torch.randn((1, c), generator=g, device=dev).to(torch.bfloat16)
            for name, c in (("attn", 8192), ("o", 8192), ("mlp", 8192), ("down", 28672))}


# which input each matrix of a layer (q, k, v, o, gate, up, down) takes
LAYER_X = ("attn", "attn", "attn", "o", "mlp", "mlp", "down")


def layer_gemv_calls(nf4, Ws, xs, ys, form):
    """One layer's decode GEMV.  form "decode": batched launches over the
    matrices that share their input (q|k|v, o, gate|up, down); "single":
    seven nf4_gemv launches; "one": one nf4_gemv_batched call (one launch)
    over all seven."""
    xl = [xs[k] for k in LAYER_X]
    if form == "single":
        for W, x, y in zip(Ws, xl, ys):
            nf4.nf4_gemv(W, x, y)
    elif form == "one":
        nf4.nf4_gemv_batched(Ws, xl, ys)
    else:
        for lo, hi in ((0, 3), (3, 4), (4, 6), (6, 7)):
            nf4.nf4_gemv_batched(Ws[lo:hi], xl[lo:hi], ys[lo:hi])


def capture_layer_steps(torch, nf4, store, layers, xs, ys, form):
    """The decode GEMV of the stored layers `layers`, one after another, as
    one HIP graph: the steps run back to back with no host dispatch between
    them, as a serving loop's captured decode does."""
    def run():
        for layer in layers:
            layer_gemv_calls(nf4, store[layer], xs, ys, form)

    run()
    return capture_graph(torch, run)


def layer_gemv_variants(torch, nf4, store, xs, ys, stream, nbytes, passes=40):
    """The same layer GEMV issued three ways over the stored layers: one graph
    of `passes` steps (a different layer each step) per form, timed with HIP
    events around the replay; mean per step."""
    res = {}
    L = len(store)
    layers = [(37 * k) % L for k in range(passes)]
    for form, what in (("single", "seven nf4_gemv launches"),
                       ("decode", "q|k|v, o, gate|up, down as four nf4_gemv_batched launches"),
                       ("one", "one nf4_gemv_batched call over the seven (one launch)")):
        graph = capture_layer_steps(torch, nf4, store, layers, xs, ys, form)
        graph.replay()
        torch.cuda.synchronize()
        t = EventTimer(torch, stream)
        s = t.start()
        graph.replay()
        t.stop(s)
        torch.cuda.synchronize()
        us = t.mean_us() / passes
        res[form] = {"what": what, "us_per_step": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "frac_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del graph
    return res


LEGS = ("hbm", "c1", "c2-step", "gemv-decode", "gemv-mlp", "gemv-70b", "stack-70b", "layer-gemv", "layer-forms", "gemm",
        "qlora-backward", "lora-merge")


def extra_legs(torch, nf4, syn, dev, stream, EventTimer, only=None):
    """GEMV alone from HBM (decode), the Llama-8B MLP and 70B-layer GEMVs, and
    the QLoRA forward GEMM; `only` runs a single one of LEGS."""
    res = {}
    g = torch.Generator(device=dev)
    if only in (None, "hbm"):
        res.update(leg_hbm_calibration(torch, dev, stream, EventTimer))
    if only in (None, "c1"):
        res.update(leg_c1(torch, nf4, syn, dev, stream, EventTimer))
    if only in (None, "c2-step"):
        res.update(leg_c2_step(torch, nf4, syn, dev, stream))
    if only in (None, "gemv-decode"):
        res.update(leg_gemv_decode(torch, nf4, syn, dev, stream, EventTimer, g))
    if only in (None, "gemv-mlp", "gemv-70b"):
        res.update(legs_gemv_pools(torch, nf4, dev, stream, EventTimer, g, only))
    if only == "stack-70b":
        res.update(leg_stack_70b(torch, nf4, syn, dev, stream, EventTimer))
    if only == "layer-forms":
        res.update(leg_layer_forms(torch, nf4, syn, dev, stream, EventTimer))
    if only == "layer-gemv":
        res.update(leg_layer_gemv(torch, nf4, syn, dev, stream, EventTimer))
    if only in (None, "gemm"):
        res.update(leg_gemm(torch, nf4, dev, stream, EventTimer, g))
    if only in (None, "qlora-backward"):
        res.update(leg_qlora_backward(torch, nf4, dev, stream, EventTimer, g))
    if only in (None, "lora-merge"):
        res.update(leg_lora_merge(torch, nf4, dev, stream, EventTimer, g))
    return res


def warm_up(torch, fn, calls=10, seconds=0.5):
    """Runs fn at least `calls` times and for at least `seconds` of wall time
    (the GPU's clock and power settle within a few hundred milliseconds of
    sustained matrix-core load; timing starts after that)."""
    t0 = time.perf_counter()
    k = 0
    while k < calls or time.perf_counter() - t0 < seconds:
        fn()
        k += 1
        if k % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def _median_call(torch, stream, EventTimer, fn, reps=30, warm=5, warm_s=0.0):
    warm_up(torch, fn, calls=warm, seconds=warm_s)
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
    us_dx = _median_call(torch, stream, EventTimer, lambda: nf4.nf4_gemm_dx(W, dY, dX, A, B, s_l, ws_dx), warm_s=0.5)
    us_g = _median_call(torch, stream, EventTimer,
                        lambda: nf4.nf4_lora_grads(X, dY, A, B, s_l, da=dA, db=dB, workspace=ws_g))
    fl_dx = 2.0 * M * N * K + 2.0 * M * N * r + 2.0 * M * r * K
    tf = fl_dx / (us_dx * 1e-6) / 1e12
    Wd = nf4.nf4_dequantize(W, out_dtype=torch.bfloat16)
    us_lib = _median_call(torch, stream, EventTimer, lambda: torch.matmul(dY, Wd), warm_s=0.5)
    del Wd
    return {"qlora_backward": {
        "workload": "dY 4096x14336 bf16, NF4(DQ) W 14336x4096, LoRA r=16 alpha=32: dX, dA, dB",
        "gemm_dx_us": round(us_dx, 1),
        "gemm_dx_TFLOPs": round(tf, 1),
        "gemm_dx_frac_mfma_bf16_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "lora_grads_us": round(us_g, 1),
        "timing": "medians of 30 calls after at least 5 warm-up calls and 0.5 s (dX call includes its LoRA prep; grads "
                  "include both thin products)",
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


def build_stack_70b(torch, nf4, syn, dev, stream, EventTimer, layers=80):
    """The 70B-shaped stack.  Layer by layer the seven bf16 weights (q, k, v,
    o, gate, up, down) are drawn on the device (untimed) and then quantized
    and double-quantized into a persistent NF4 store (timed: one HIP graph per
    layer of one nf4_quantize_batched launch over the seven weights and one
    nf4_double_quant_batched call over their seven scale arrays).  Returns the
    store and the stack's figures."""
    layers = max(1, min(int(layers), 80))
    print(f"[bench] 70B stack: {layers} layers", file=sys.stderr, flush=True)
    LAYER_70B = [syn.C5_SHAPES[name] for name in syn.C5_ORDER]
    src = [torch.empty(sh, dtype=torch.bfloat16, device=dev) for sh in LAYER_70B]
    nbs = [r * c // 64 for r, c in LAYER_70B]
    absmax = [torch.empty(nb, dtype=torch.float32, device=dev) for nb in nbs]
    dq_ws = torch.empty(nf4.lib().nf4_double_quant_batched_workspace(len(nbs)), dtype=torch.uint8, device=dev)
    store, t = [], EventTimer(torch, stream)
    for layer in range(layers):
        Ws = []
        for (r, c), nb in zip(LAYER_70B, nbs):
            Ws.append(nf4.NF4Weight(torch.empty(r * c // 2, dtype=torch.uint8, device=dev), r, c,
                                    qabsmax=torch.empty(nb, dtype=torch.int8, device=dev),
                                    absmax2=torch.empty(-(-nb // 256), dtype=torch.float32, device=dev),
                                    mean=torch.empty(1, dtype=torch.float32, device=dev)))

        def run():
            nf4.nf4_quantize_batched(src, outs=[(W.packed, am) for W, am in zip(Ws, absmax)])
            nf4.nf4_double_quant_batched(absmax, outs=[(W.qabsmax, W.absmax2, W.mean) for W in Ws], workspace=dq_ws)

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
    g_bytes = sum(step_bytes(r, c)["gemv"] for r, c in LAYER_70B)
    return store, {
        "workload": f"{layers} layers of q,o 8192x8192, k,v 1024x8192, gate,up 28672x8192, down 8192x28672, bf16 "
                    "N(0,0.02) drawn per layer on the device; NF4 + int8 double quant into a persistent store",
        "layers": layers,
        "quantize_dq_us_per_layer": round(sum(q_us) / layers, 1),
        "quantize_dq_input_GBps": round(2 * n_layer * layers / total_s / 1e9, 1),
        "quantize_dq_algorithmic_GBps": round(alg_layer * layers / total_s / 1e9, 1),
        "quantize_dq_frac_hbm_peak": round(alg_layer * layers / total_s / 1e9 / HBM_PEAK_GBS, 4),
        "nf4_store_GB": round(layers * g_bytes / 1e9, 2),
        "timing": "HIP events around each layer's graph: one nf4_quantize_batched call over the seven weights, "
                  "then one nf4_double_quant_batched call over their seven scale arrays",
    }


def leg_layer_gemv(torch, nf4, syn, dev, stream, EventTimer, layers=6, passes=12):
    """The headline step alone (for counter runs): a store of a few layers
    (2.6 GB, far beyond the last-level cache) and `passes` steps of the
    decode GEMV in the benchmark's launch form as one graph, a different
    layer each step."""
    store, _ = build_stack_70b(torch, nf4, syn, dev, stream, EventTimer, layers)
    shapes = [syn.C5_SHAPES[name] for name in syn.C5_ORDER]
    xs = layer_inputs(torch, dev)
    ys = [torch.empty((1, r), dtype=torch.bfloat16, device=dev) for r, _ in shapes]
    graph = capture_layer_steps(torch, nf4, store, [k % layers for k in range(passes)], xs, ys, "one")
    torch.cuda.synchronize()
    t = EventTimer(torch, stream)
    s = t.start()
    graph.replay()
    t.stop(s)
    torch.cuda.synchronize()
    nbytes = sum(step_bytes(r, c)["gemv"] for r, c in shapes)
    us = t.mean_us() / passes
    del graph, store
    return {"layer_gemv": {"layers": layers, "passes": passes, "us_per_step": round(us, 2),
                           "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}}


def leg_layer_forms(torch, nf4, syn, dev, stream, EventTimer, layers=6):
    """The layer's decode GEMV issued three ways (seven single launches, the
    decode order's four batched launches, one batched launch) over a store of
    a few layers, a different layer each step.  Kept out of the default run,
    whose kernel trace then holds the one-launch form alone."""
    store, _ = build_stack_70b(torch, nf4, syn, dev, stream, EventTimer, layers)
    shapes = [syn.C5_SHAPES[name] for name in syn.C5_ORDER]
    xs = layer_inputs(torch, dev)
    ys = [torch.empty((1, r), dtype=torch.bfloat16, device=dev) for r, _ in shapes]
    nbytes = sum(step_bytes(r, c)["gemv"] for r, c in shapes)
    res = layer_gemv_variants(torch, nf4, store, xs, ys, stream, nbytes)
    del store
    return {"gemv_layer_70b_launch_forms": {"layers": layers, **res}}


def leg_stack_70b(torch, nf4, syn, dev, stream, EventTimer, layers=80, gemv_passes=20):
    """The stack alone (for profiling): the store, then the decode GEMV over
    one layer's seven matrices, a different stored layer on each pass."""
    store, stack = build_stack_70b(torch, nf4, syn, dev, stream, EventTimer, layers)
    shapes = [syn.C5_SHAPES[name] for name in syn.C5_ORDER]
    g = torch.Generator(device=dev)
    g.manual_seed(5_000_009)
    xs = {c: torch.randn((1, c), generator=g, device=dev).to(torch.bfloat16) for _, c in shapes}
    ys = [torch.empty((1, r), dtype=torch.bfloat16, device=dev) for r, _ in shapes]
    tg = EventTimer(torch, stream)
    for k in range(gemv_passes):
        Ws = store[(37 * k) % len(store)]
        s = tg.start()
        for W, yy in zip(Ws, ys):
            nf4.nf4_gemv(W, xs[W.cols], yy)
        tg.stop(s)
    torch.cuda.synchronize()
    g_bytes = sum(step_bytes(r, c)["gemv"] for r, c in shapes)
    g_med = tg.median_us()
    del store
    stack["gemv_layer_eager"] = {"passes": gemv_passes, "median_us": round(g_med, 2),
                                 "GBps": round(g_bytes / (g_med * 1e-6) / 1e9, 1)}
    return {"stack_70b": stack}


def stream_read_gbps(torch, dev, stream, EventTimer, nbytes=4 << 30):
    """The best of a few launch shapes, with plain or non-temporal loads, of
    the streaming-read kernel (libnf4_calib.so, built beside the library)
    over a 4 GiB buffer: what the memory system gives a read-only kernel
    here.  Returns GB/s and the shape, or None when the calibration library
    is missing."""
    import ctypes
    path = os.path.join(ROOT, "dequant_matmul_nf4_amd", "libnf4_calib.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    f = L.nf4_calib_stream_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint32,
                  ctypes.c_void_p, ctypes.c_void_p]
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(0x01010101)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.zeros(16 * cus, dtype=torch.int32, device=dev)
    best = None
    for per_cu in (2, 4, 8, 16):
        for unroll in (4, 8):
            for nt in (0, 1):
                grid = per_cu * cus

                def call():
                    rc = f(buf.data_ptr(), nbytes, grid, unroll, nt, 0x5A5A5A5A, out.data_ptr(), stream.cuda_stream)
                    if rc != 0:
                        raise RuntimeError(f"nf4_calib_stream_read failed: {rc}")

                us = _median_call(torch, stream, EventTimer, call, reps=10, warm=2)
                gbs = nbytes / (us * 1e-6) / 1e9
                if best is None or gbs > best["GBps"]:
                    best = {"GBps": round(gbs, 1), "us": round(us, 1), "workgroups": grid, "threads": 512,
                            "loads_in_flight_per_lane": unroll, "nontemporal": bool(nt)}
    del buf, out
    return best


def leg_hbm_calibration(torch, dev, stream, EventTimer):
    """What the memory system gives on this GPU, as the measured-achievable
    context for the HBM-bound kernels: torch's device copy (read + write) and
    full reduction (read only) over 2 GiB, and a plain streaming-read kernel
    of our own over 4 GiB."""
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
    sr = stream_read_gbps(torch, dev, stream, EventTimer)
    if sr:
        out["stream_read"] = sr
    return {"hbm_calibration": {"what": "torch copy_ (2 GiB read + 2 GiB write) and sum (2 GiB read), median of 10; "
                                        "stream_read: our plain read kernel over 4 GiB, best launch shape, median of 10",
                                **out}}


def leg_c1(torch, nf4, syn, dev, stream, EventTimer):
    """The 1024 x 1024 float32 weight without double quantization: quantize,
    dequantize (float32 out) and the GEMV with one bf16 x, each a median of
    200 event-timed calls.  4.8 MB sit in the caches, so these are latencies,
    not bandwidths."""
    print("[bench] C1 round trip", file=sys.stderr, flush=True)
    inp = syn.c1_inputs()
    w = torch.from_numpy(inp["w_f32"]).to(dev)
    x = inp["x"].to(dev)
    packed, absmax = nf4.nf4_quantize(w)
    W = nf4.NF4Weight(packed, 1024, 1024, absmax=absmax)
    out = torch.empty((1024, 1024), dtype=torch.float32, device=dev)
    y = torch.empty((1, 1024), dtype=torch.float32, device=dev)
    res = {}
    for name, fn in (("quantize_us", lambda: nf4.nf4_quantize(w, packed, absmax)),
                     ("dequantize_us", lambda: nf4.nf4_dequantize(W, out=out)),
                     ("gemv_us", lambda: nf4.nf4_gemv(W, x, y))):
        res[name] = round(_median_call(torch, stream, EventTimer, fn, reps=200, warm=10), 2)
    return {"c1_round_trip": {"workload": "1024x1024 fp32 N(0,0.02), no double quant; x bf16 [1, 1024]",
                              "timing": "median of 200 event-timed calls each (includes the launch)", **res}}


def leg_c2_step(torch, nf4, syn, dev, stream, P=16, steps=20):
    """The 4096^2 attention projection with outliers: nf4_quantize of every
    weight of a pool of P, nf4_double_quant of every absmax, nf4_gemv on
    every weight, as three HIP graphs per pass; per-kernel averages from
    events between the graphs."""
    print(f"[bench] 4096x4096 quantize + double quant + GEMV composite, pool {P}", file=sys.stderr, flush=True)
    rows = cols = 4096
    ws = [syn.c2_weight(pool_index=i).to(dev) for i in range(P)]
    x = syn.c2_inputs()["x"].to(dev)
    n = rows * cols
    nb = n // 64
    bufs = [dict(packed=torch.empty(n // 2, dtype=torch.uint8, device=dev),
                 absmax=torch.empty(nb, dtype=torch.float32, device=dev),
                 q=torch.empty(nb, dtype=torch.int8, device=dev),
                 s2=torch.empty(-(-nb // 256), dtype=torch.float32, device=dev),
                 mean=torch.empty(1, dtype=torch.float32, device=dev),
                 y=torch.empty((1, rows), dtype=torch.bfloat16, device=dev)) for _ in range(P)]
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

    for f in (run_quantize, run_double_quant, run_gemv):
        f()
    torch.cuda.synchronize()
    graphs = [capture_graph(torch, f) for f in (run_quantize, run_double_quant, run_gemv)]
    for _ in range(3):
        for gr in graphs:
            gr.replay()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        for j, gr in enumerate(graphs):
            evs[k][j].record(stream)
            gr.replay()
        evs[k][3].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    sb = step_bytes(rows, cols)
    phase_us = [1e3 * sum(e[j].elapsed_time(e[j + 1]) for e in evs) / (steps * P) for j in range(3)]
    del graphs, ws, bufs
    return {"c2_step": {
        "workload": "4096x4096 bf16 N(0,0.02) + 0.1% outliers x20, pool of 16 (512 MiB of bf16); per pass: "
                    "nf4_quantize, nf4_double_quant, nf4_gemv (m=1) of every weight, three HIP graphs",
        "GBps": round(P * sum(sb.values()) * steps / elapsed / 1e9, 1),
        "quantize_us": round(phase_us[0], 3),
        "quantize_GBps": round(sb["quantize"] / (phase_us[0] * 1e-6) / 1e9, 1),
        "double_quant_us": round(phase_us[1], 3),
        "gemv_us": round(phase_us[2], 3),
        "gemv_note": "the GEMV reads codes the quantizer has just written (partly cache-resident)",
    }}


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


def gemv_mlp_batched(torch, nf4, dev, stream, EventTimer, g, reps=10, triples=6):
    """The Llama-8B MLP decode step at m = 1 as a caller would issue it: gate
    and up (which share x) in one nf4_gemv_batched launch, then down; six
    distinct weight triples per pass, as the single-call leg."""
    shapes = [(14336, 4096), (14336, 4096), (4096, 14336)]
    Wt = []
    for t in range(triples):
        ws = []
        for i, (r_, c_) in enumerate(shapes):
            g.manual_seed(9_000 + 3 * t + i)
            w = (torch.randn((r_, c_), generator=g, device=dev) * 0.02).to(torch.bfloat16)
            ws.append(nf4.quantize_weight(w, double_quant=True))
            del w
        Wt.append(ws)
    x_in = torch.randn((1, 4096), generator=g, device=dev).to(torch.bfloat16)
    x_h = torch.randn((1, 14336), generator=g, device=dev).to(torch.bfloat16)
    ys = [[torch.empty((1, r_), dtype=torch.bfloat16, device=dev) for r_, _ in shapes] for _ in range(triples)]

    def run():
        for ws, yy in zip(Wt, ys):
            nf4.nf4_gemv_batched(ws[:2], [x_in, x_in], yy[:2])
            nf4.nf4_gemv(ws[2], x_h, yy[2])

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
    nbytes = triples * sum(step_bytes(r_, c_)["gemv"] for r_, c_ in shapes)
    del Wt
    return {"workload": "Llama-8B MLP at m=1, 6 distinct triples (545 MB) per pass: gate and up in one nf4_gemv_batched "
                        "launch (they share x), then down", "m": 1, "us_per_pass": round(total_us, 2),
            "GBps": round(nbytes / (total_us * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (total_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


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
        res["gemv_mlp_8b_batched"] = gemv_mlp_batched(torch, nf4, dev, stream, EventTimer, g, reps=10)
    if only in (None, "gemv-70b"):
        layer = [(8192, 8192), (1024, 8192), (1024, 8192), (8192, 8192), (28672, 8192), (28672, 8192),
                 (8192, 28672)]
        res["gemv_layer_70b"] = gemv_pool(layer, 10, "70B-shaped layer q,k,v,o,gate,up,down NF4+DQ, M=1 (442 MB)")
        res["gemv_layer_70b_fp8_scales"] = gemv_pool(
            layer, 10, "the same layer with float8 (E4M3) second-level scales, M=1", dq_type="fp8")
        res["gemv_layer_70b_m16"] = gemv_pool(layer, 10, "the same layer at M=16 (seven nf4_gemv calls)", m=16)
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
    # 50 event-timed calls after at least 10 warm-up calls and 0.5 s
    warm_up(torch, lambda: nf4.nf4_gemm(W, X, Y, A, B, 2.0, wsb))
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
    us_mean = t.mean_us()
    # the base product alone: one k_gemm launch per call
    us_base = _median_call(torch, stream, EventTimer, lambda: nf4.nf4_gemm(W, X, Y), reps=reps, warm=5, warm_s=0.5)
    fl_base = 2.0 * M * N * K
    res["gemm_qlora_forward"] = {
        "workload": "X 4096x4096 bf16 . NF4(DQ) W 14336x4096^T + LoRA r=16 alpha=32",
        "flops": flops,
        "us": round(us, 1),
        "us_mean": round(us_mean, 1),
        "TFLOPs": round(flops / (us_mean * 1e-6) / 1e12, 1),
        "TFLOPs_median": round(tf, 1),
        "frac_mfma_bf16_peak": round(flops / (us_mean * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "timing": f"HIP events around each of {reps} calls (LoRA prep + GEMM) after at least 10 warm-up calls and "
                  "0.5 s; TFLOPs from the mean",
        "no_lora": {"us": round(us_base, 1), "TFLOPs": round(fl_base / (us_base * 1e-6) / 1e12, 1),
                    "what": "nf4_gemm without adapters: the k_gemm launch alone, median of 50"},
    }
    # Calibration only (not part of the path): the vendor library's plain bf16
    # GEMM of the same shape on an already dequantized weight, no LoRA.
    Wd = nf4.nf4_dequantize(W, out_dtype=torch.bfloat16)
    warm_up(torch, lambda: torch.nn.functional.linear(X, Wd))
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


def cpu_baseline(np, syn, torch, dev, min_seconds: float = 10.0):
    """The CPU oracle (as it stands) on a bounded sample of the workload.

    The headline leg: the oracle's decode GEMV of layer 0's k and v matrices
    (1024 x 8192 each): dequantize from the oracle's own NF4 + double-quant
    form, then the float64 product with x (numpy BLAS on every allowed core),
    repeated for at least `min_seconds`; GB/s counted with the same
    algorithmic bytes as the GPU.  The stack leg: the oracle's quantize +
    double quant of the k matrix of layers 0, 41 and 79, its per-weight rate
    extrapolated to the 80-layer stack (labelled so)."""
    import oracle
    print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
    shapes = {name: syn.C5_SHAPES[name] for name in ("k", "v")}
    g = torch.Generator(device=dev)
    g.manual_seed(5_000_009)
    xs = {c: torch.randn((1, c), generator=g, device=dev).to(torch.bfloat16) for _, c in syn.C5_SHAPES.values()}
    forms = []
    for name, (rows, cols) in shapes.items():
        w = syn.bf16_to_f32(syn.c5_weight_device(0, name, device=dev)).reshape(-1)
        p, a = oracle.quantize(w)
        q, s2, mu = oracle.double_quant(a)
        forms.append((rows, cols, p, q, s2, mu, syn.bf16_to_f32(xs[cols])))
    reps = 0
    t0 = time.perf_counter()
    while True:
        for rows, cols, p, q, s2, mu, x in forms:
            wd = oracle.bf16_bits_to_f32(oracle.dequantize(p, rows * cols, qabsmax=q, absmax2=s2, mean=mu, out="bf16"))
            oracle.matmul_ref(x, wd.reshape(rows, cols))
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    nbytes = sum(step_bytes(r, c)["gemv"] for r, c in shapes.values())
    # quantize + double quant sample, extrapolated to the whole stack
    qt, nq = 0.0, 0
    for layer in (0, 41, 79):
        w = syn.bf16_to_f32(syn.c5_weight_device(layer, "k", device=dev)).reshape(-1)
        t1 = time.perf_counter()
        p, a = oracle.quantize(w)
        oracle.double_quant(a)
        qt += time.perf_counter() - t1
        nq += w.size
    n_stack = 80 * sum(r * c for r, c in syn.C5_SHAPES.values())
    cores = len(os.sched_getaffinity(0))
    return {
        "value": round(reps * nbytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{reps} passes of the oracle's decode GEMV (dequantize + float64 product) over layer 0's k and v "
                  f"matrices (1024x8192 each, {nbytes} algorithmic bytes per pass) of the 70B-shaped stack; "
                  "dequantize runs on one core, the product on numpy's BLAS threads",
        "seconds": round(dt, 2),
        "quantize_dq_sample": {
            "what": "oracle quantize + double quant of the k matrix (1024x8192) of layers 0, 41, 79, one core",
            "seconds": round(qt, 2),
            "input_GBps": round(2 * nq / qt / 1e9, 5),
            "extrapolated_80_layer_stack_s": round(qt / nq * n_stack, 1),
            "note": "extrapolated: the per-weight time of the sample times the stack's 68.4 G weights",
        },
    }


if __name__ == "__main__":
    sys.exit(main())
