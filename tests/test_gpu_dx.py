"""GPU parity of nf4_gemm_dx (the input gradient through the frozen base,
dX = dY . deq(W) + s . (dY . B) . A) against the oracle's float64
backward_ref on its bf16-dequantized weights: relative Frobenius error
<= 1e-2 (MATMUL_RTOL).  The full C4 backward is checked on sampled columns
of dX, each from the oracle's dequantization of the blocks it needs."""

from __future__ import annotations

import numpy as np
import pytest

import dequant_matmul_nf4_amd as nf4
import oracle
import synthetic as syn
from tests.gpu_common import MATMUL_RTOL, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _full_oracle_wdeq(w_f32: np.ndarray, dq: bool) -> np.ndarray:
    p, a = oracle.quantize(w_f32.reshape(-1))
    if dq:
        q, s2, mean = oracle.double_quant(a)
        bits = oracle.dequantize(p, w_f32.size, qabsmax=q, absmax2=s2, mean=mean, out="bf16")
    else:
        bits = oracle.dequantize(p, w_f32.size, absmax=a, out="bf16")
    return oracle.bf16_bits_to_f32(bits).reshape(w_f32.shape)


def _f64(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def _run(m, rows, cols, r, dq, seed):
    torch = need_gpu()
    w = syn.normal_f32((rows, cols), 0.02, seed)
    dyb = syn.to_bf16(syn.normal_f32((m, rows), 1.0, seed + 1))
    W = nf4.quantize_weight(to_dev(w), double_quant=dq)
    a = b = None
    s = 0.0
    if r:
        a = syn.to_bf16(syn.normal_f32((r, cols), 0.02, seed + 2))
        b = syn.to_bf16(syn.normal_f32((rows, r), 0.02, seed + 3))
        s = 32.0 / r
    dx = nf4.nf4_gemm_dx(W, dyb.to("cuda"), lora_a=None if a is None else a.to("cuda"),
                         lora_b=None if b is None else b.to("cuda"), lora_scale=s)
    torch.cuda.synchronize()
    ref, _, _ = oracle.backward_ref(syn.bf16_to_f32(dyb), _full_oracle_wdeq(w, dq),
                                    lora_a=None if a is None else syn.bf16_to_f32(a),
                                    lora_b=None if b is None else syn.bf16_to_f32(b), lora_scale=s)
    e = oracle.rel_frobenius(_f64(dx), ref)
    say(f"  rel err {e:.2e}")
    return e


# ragged m (tile 256), rows not a multiple of the 64-row step, cols not a
# multiple of the 256-column tile
@pytest.mark.parametrize("m,rows,cols", [(1, 64, 64), (37, 200, 128), (130, 136, 192), (256, 256, 512),
                                         (300, 520, 1024), (513, 1032, 320)])
@pytest.mark.parametrize("lora", [0, 1, 16])
@pytest.mark.parametrize("dq", [False, True])
def test_dx_small(m, rows, cols, lora, dq):
    say("gemm_dx", m, rows, cols, "lora", lora, "dq" if dq else "plain")
    assert _run(m, rows, cols, lora, dq, m + 3 * rows + cols) <= MATMUL_RTOL


@pytest.mark.parametrize("m,rows,cols,r", [(513, 304, 320, 64), (100, 264, 64, 33), (33, 256, 128, 17),
                                           (260, 8, 256, 48)])
def test_dx_lora_ranks(m, rows, cols, r):
    """Largest rank, ranks that are not a multiple of 16, ragged shapes, a
    weight with a single partial reduction step."""
    say("gemm_dx lora rank", r, "shape", m, rows, cols)
    assert _run(m, rows, cols, r, True, 70 + r) <= MATMUL_RTOL


def test_dx_closed_forms():
    """A one-hot row of dY returns a dequantized weight row exactly (one
    nonzero product, rounded once to bf16); with B = 0 the adapter term adds
    nothing, bit for bit."""
    say("gemm_dx closed forms")
    torch = need_gpu()
    rows, cols, m = 200, 320, 300
    w = syn.normal_f32((rows, cols), 0.02, 21)
    W = nf4.quantize_weight(to_dev(w), double_quant=True)
    wdeq = nf4.nf4_dequantize(W, out_dtype=torch.bfloat16)
    e = torch.zeros((m, rows), dtype=torch.bfloat16, device="cuda")
    pick = [(i * 7) % rows for i in range(m)]
    for i in range(m):
        e[i, pick[i]] = 1.0
    dxe = nf4.nf4_gemm_dx(W, e)
    dyb = syn.to_bf16(syn.normal_f32((m, rows), 1.0, 22)).to("cuda")
    a = syn.to_bf16(syn.normal_f32((16, cols), 0.02, 23)).to("cuda")
    zb = torch.zeros((rows, 16), dtype=torch.bfloat16, device="cuda")
    d0 = nf4.nf4_gemm_dx(W, dyb)
    d1 = nf4.nf4_gemm_dx(W, dyb, lora_a=a, lora_b=zb, lora_scale=2.0)
    torch.cuda.synchronize()
    for i in range(m):
        assert torch.equal(dxe[i], wdeq[pick[i]])
    assert torch.equal(d0, d1)


def test_dx_is_the_adjoint_of_the_forward():
    """<dY, gemm(X)> = <gemm_dx(dY), X> for the same weight and adapters (the
    backward is the transpose of the forward), up to the bf16 outputs."""
    say("gemm_dx adjoint")
    torch = need_gpu()
    m, rows, cols, r = 96, 520, 384, 16
    w = syn.normal_f32((rows, cols), 0.02, 31)
    W = nf4.quantize_weight(to_dev(w), double_quant=True)
    x = syn.to_bf16(syn.normal_f32((m, cols), 1.0, 32)).to("cuda")
    dy = syn.to_bf16(syn.normal_f32((m, rows), 1.0, 33)).to("cuda")
    a = syn.to_bf16(syn.normal_f32((r, cols), 0.05, 34)).to("cuda")
    b = syn.to_bf16(syn.normal_f32((rows, r), 0.05, 35)).to("cuda")
    y = nf4.nf4_gemm(W, x, lora_a=a, lora_b=b, lora_scale=2.0)
    dx = nf4.nf4_gemm_dx(W, dy, lora_a=a, lora_b=b, lora_scale=2.0)
    torch.cuda.synchronize()
    lhs = float((_f64(dy) * _f64(y)).sum())
    rhs = float((_f64(dx) * _f64(x)).sum())
    scale = np.linalg.norm(_f64(dy)) * np.linalg.norm(_f64(y))
    say(f"  <dy,y> {lhs:.6e} <dx,x> {rhs:.6e}")
    assert abs(lhs - rhs) <= 1e-2 * scale
