"""Every entry point captured into a HIP graph and replayed several times,
with eager work and synchronizations between the replays: each replay must
reproduce the eager results bit for bit (the kernels are deterministic and
record no memset nodes)."""

from __future__ import annotations

import pytest

import dequant_matmul_nf4_amd as nf4
import synthetic as syn
from tests.gpu_common import need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    torch = need_gpu()
    rows, cols, m, r = 320, 512, 40, 16
    say("graph capture", rows, cols, m, r)
    w = to_dev(syn.normal_f32((rows, cols), 0.02, 91)).to(torch.bfloat16)
    x1 = syn.to_bf16(syn.normal_f32((1, cols), 1.0, 92)).to("cuda")
    xm = syn.to_bf16(syn.normal_f32((m, cols), 1.0, 93)).to("cuda")
    a = syn.to_bf16(syn.normal_f32((r, cols), 0.01, 94)).to("cuda")
    b = syn.to_bf16(syn.normal_f32((rows, r), 0.01, 95)).to("cuda")
    n, nb = rows * cols, rows * cols // 64

    out = dict(
        packed=torch.empty(n // 2, dtype=torch.uint8, device="cuda"),
        absmax=torch.empty(nb, dtype=torch.float32, device="cuda"),
        q=torch.empty(nb, dtype=torch.int8, device="cuda"),
        s2=torch.empty(-(-nb // 256), dtype=torch.float32, device="cuda"),
        mean=torch.empty(1, dtype=torch.float32, device="cuda"),
        deq=torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda"),
        y1=torch.empty((1, rows), dtype=torch.float32, device="cuda"),
        y4=torch.empty((4, rows), dtype=torch.bfloat16, device="cuda"),
        ym=torch.empty((m, rows), dtype=torch.bfloat16, device="cuda"),
        dx=torch.empty((m, cols), dtype=torch.bfloat16, device="cuda"),
        da=torch.empty((r, cols), dtype=torch.float32, device="cuda"),
        db=torch.empty((rows, r), dtype=torch.float32, device="cuda"),
        merged=torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda"),
        q8=torch.empty(nb, dtype=torch.uint8, device="cuda"),
        s28=torch.empty(-(-nb // 256), dtype=torch.float32, device="cuda"),
        mean8=torch.empty(1, dtype=torch.float32, device="cuda"),
        y8=torch.empty((1, rows), dtype=torch.float32, device="cuda"),
    )
    dy = syn.to_bf16(syn.normal_f32((m, rows), 1.0, 96)).to("cuda")
    dq_ws = torch.empty(nf4.nf4_double_quant_workspace(nb), dtype=torch.uint8, device="cuda")
    mm_ws = torch.empty(nf4.nf4_gemm_workspace(m, rows, r), dtype=torch.uint8, device="cuda")
    dx_ws = torch.empty(nf4.nf4_gemm_dx_workspace(m, rows, r), dtype=torch.uint8, device="cuda")
    gr_ws = torch.empty(nf4.nf4_lora_grads_workspace(m, rows, cols, r), dtype=torch.uint8, device="cuda")
    W = nf4.NF4Weight(out["packed"], rows, cols, qabsmax=out["q"], absmax2=out["s2"], mean=out["mean"])
    W8 = nf4.NF4Weight(out["packed"], rows, cols, qabsmax=out["q8"], absmax2=out["s28"], mean=out["mean8"],
                       dq_type=nf4.NF4_DQ_FP8)

    def path():
        nf4.nf4_quantize(w, out["packed"], out["absmax"])
        nf4.nf4_double_quant(out["absmax"], out["q"], out["s2"], out["mean"], dq_ws)
        nf4.nf4_dequantize(W, out["deq"])
        nf4.nf4_gemv(W, x1, out["y1"])
        nf4.nf4_gemv(W, xm[:4], out["y4"])
        nf4.nf4_gemm(W, xm, out["ym"], a, b, 2.0, mm_ws)
        nf4.nf4_gemm_dx(W, dy, out["dx"], a, b, 2.0, dx_ws)
        nf4.nf4_lora_grads(xm, dy, a, b, 2.0, da=out["da"], db=out["db"], workspace=gr_ws)
        nf4.nf4_lora_merge(W, a, b, 2.0, out=out["merged"])
        nf4.nf4_double_quant(out["absmax"], out["q8"], out["s28"], out["mean8"], dq_ws, fp8=True)
        nf4.nf4_gemv(W8, x1, out["y8"])

    path()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in out.items()}

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        path()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in out.values():
            v.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            assert torch.equal(v, eager[k]), (rep, k)
        del junk
