"""Full-size parity of the matmul paths, on every output.

The QLoRA forward GEMM and its input gradient at 4096 x 4096 x 14336
(LoRA r = 16, alpha = 32), the Llama-8B MLP decode GEMVs (14336 x 4096 and
4096 x 14336 at m = 1, 2, 4 and 16), and GEMMs of intermediate size whose
persistent workgroups take several tiles each (with and without the XCD tile
order), are compared output by output with the oracle's float64 product of
its own dequantized weight (bitsandbytes tool page, "How it works", Step 5:
dequantize, then multiply; tutorial page "QLoRA: Fine-Tuning a 4-bit Model":
adapters on the frozen base, scaled).  Bounds: gpu_common.check_full_product
(relative Frobenius error <= 1e-2 over the whole output and over every tile,
plus a per-element bound from the arithmetic)."""

from __future__ import annotations

import numpy as np
import pytest

import dequant_matmul_nf4_amd as nf4
import oracle
import synthetic as syn
from tests.gpu_common import (check_full_product, need_gpu, oracle_wdeq_full, say, syn_c4, to_dev)

pytestmark = pytest.mark.gpu

GEMM_TILE = (256, 256)      # output tile of nf4_gemm (rows of x, rows of W)
DX_TILE = (256, 256)        # output tile of nf4_gemm_dx
GEMV_TILE = (1, 64)         # groups of 64 outputs of one x row
LORA_SPLIT_REL = 2.0 ** -16  # s T carried as two bf16 parts


def _f64(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def _abs_product(x, w, a=None, b=None, s=0.0):
    """|x| |w|^T (+ |s| (|x| |a|^T) |b|^T): the sum of the magnitudes of the
    terms each output adds up, for the per-element bound."""
    sabs = np.abs(x).astype(np.float64) @ np.abs(w).astype(np.float64).T
    if a is not None:
        t = np.abs(x).astype(np.float64) @ np.abs(a).astype(np.float64).T
        sabs += abs(s) * (t @ np.abs(b).astype(np.float64).T)
    return sabs


def test_gemm_c4_every_output():
    """X [4096, 4096] . NF4(DQ) W [14336, 4096]^T + 2 (X A^T) B^T, r = 16:
    all 58.7 M outputs, all 896 tiles; a second call is bit-identical."""
    say("gemm C4 every output")
    torch = need_gpu()
    inp = syn_c4()
    x, wt, a, b = inp["x"], inp["w"], inp["a"], inp["b"]
    s = inp["alpha"] / inp["r"]
    W = nf4.quantize_weight(wt.to("cuda"), double_quant=True)
    ad, bd, xd = a.to("cuda"), b.to("cuda"), x.to("cuda")
    y = nf4.nf4_gemm(W, xd, lora_a=ad, lora_b=bd, lora_scale=s)
    y2 = nf4.nf4_gemm(W, xd, lora_a=ad, lora_b=bd, lora_scale=s)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    got = _f64(y)
    del y, y2
    wdeq = oracle_wdeq_full("c4")
    xf, af, bf = (syn.bf16_to_f32(t) for t in (x, a, b))
    ref = oracle.matmul_ref(xf, wdeq, af, bf, s)
    sabs = _abs_product(xf, wdeq, af, bf, s)
    check_full_product(got, ref, sabs, terms=xf.shape[1] + 64, tile=GEMM_TILE, w_rel=LORA_SPLIT_REL, label="C4 gemm")


def test_gemm_dx_c4_every_output():
    """dY [4096, 14336] . deq(W) + 2 (dY B) A for the same layer: all 16.8 M
    outputs and 256 tiles of dX; a second call is bit-identical."""
    say("gemm_dx C4 every output")
    torch = need_gpu()
    inp = syn_c4()
    wt, a, b = inp["w"], inp["a"], inp["b"]
    s = inp["alpha"] / inp["r"]
    dy = syn.c4_grad()
    W = nf4.quantize_weight(wt.to("cuda"), double_quant=True)
    ad, bd, dyd = a.to("cuda"), b.to("cuda"), dy.to("cuda")
    dx = nf4.nf4_gemm_dx(W, dyd, lora_a=ad, lora_b=bd, lora_scale=s)
    dx2 = nf4.nf4_gemm_dx(W, dyd, lora_a=ad, lora_b=bd, lora_scale=s)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx2)
    got = _f64(dx)
    del dx, dx2
    wdeq = oracle_wdeq_full("c4")
    dyf, af, bf = (syn.bf16_to_f32(t) for t in (dy, a, b))
    ref, _, _ = oracle.backward_ref(dyf, wdeq, lora_a=af, lora_b=bf, lora_scale=s)
    # sum of magnitudes: |dY| |W| + |s| (|dY| |B|) |A|
    sabs = np.abs(dyf).astype(np.float64) @ np.abs(wdeq).astype(np.float64)
    sabs += abs(s) * ((np.abs(dyf).astype(np.float64) @ np.abs(bf).astype(np.float64)) @ np.abs(af).astype(np.float64))
    check_full_product(got, ref, sabs, terms=dyf.shape[1] + 64, tile=DX_TILE, w_rel=LORA_SPLIT_REL, label="C4 dx")


@pytest.mark.parametrize("m,rows,cols,r", [
    (2304, 8192, 256, 0),     # 9 x 32 = 288 tiles (a multiple of 8: XCD tile order), > one per CU
    (2341, 8292, 320, 16),    # 10 x 33 = 330 tiles, ragged M and N, plain tile order, LoRA
    (4608, 4096, 128, 7),     # 18 x 16 = 288 tiles, rank not a multiple of 16
    (2048, 16384, 128, 0),    # 8 x 64 = 512 tiles: two whole rounds, no half tiles
    (2048, 14592, 192, 16),   # 8 x 57 = 456 tiles: a last round of 200, too many to halve
])
def test_gemm_persistent_tiles_every_output(m, rows, cols, r):
    """More tiles than compute units, so each persistent workgroup walks
    several tiles and reuses its LDS across them; checked on every output.
    On 256 compute units the first three shapes end with a round of 32 or 74
    tiles cut into 128-row halves; the last two keep every tile whole."""
    say("gemm persistent", m, rows, cols, "r", r)
    torch = need_gpu()
    w = syn.normal_f32((rows, cols), 0.02, 500 + rows)
    xb = syn.to_bf16(syn.normal_f32((m, cols), 1.0, 501 + m))
    W = nf4.quantize_weight(to_dev(w), double_quant=True)
    a = b = None
    s = 0.0
    if r:
        a = syn.to_bf16(syn.normal_f32((r, cols), 0.05, 502))
        b = syn.to_bf16(syn.normal_f32((rows, r), 0.05, 503))
        s = 32.0 / r
    y = nf4.nf4_gemm(W, xb.to("cuda"), lora_a=None if a is None else a.to("cuda"),
                     lora_b=None if b is None else b.to("cuda"), lora_scale=s)
    torch.cuda.synchronize()
    p, am = oracle.quantize(w.reshape(-1))
    q, s2, mean = oracle.double_quant(am)
    wdeq = oracle.bf16_bits_to_f32(oracle.dequantize(p, w.size, qabsmax=q, absmax2=s2, mean=mean, out="bf16")).reshape(w.shape)
    xf = syn.bf16_to_f32(xb)
    af = None if a is None else syn.bf16_to_f32(a)
    bf = None if b is None else syn.bf16_to_f32(b)
    ref = oracle.matmul_ref(xf, wdeq, af, bf, s)
    check_full_product(_f64(y), ref, _abs_product(xf, wdeq, af, bf, s), terms=cols + 128, tile=GEMM_TILE,
                       w_rel=LORA_SPLIT_REL if r else 0.0, label="gemm")


@pytest.mark.parametrize("m,rows,cols,r", [(2304, 256, 8192, 16), (600, 1032, 3200, 0)])
def test_gemm_dx_many_tiles_every_output(m, rows, cols, r):
    """Input gradient with more output tiles than compute units, and a
    ragged shape; every output."""
    say("gemm_dx many tiles", m, rows, cols, "r", r)
    torch = need_gpu()
    w = syn.normal_f32((rows, cols), 0.02, 600 + rows)
    dyb = syn.to_bf16(syn.normal_f32((m, rows), 1.0, 601 + m))
    W = nf4.quantize_weight(to_dev(w), double_quant=True)
    a = b = None
    s = 0.0
    if r:
        a = syn.to_bf16(syn.normal_f32((r, cols), 0.05, 602))
        b = syn.to_bf16(syn.normal_f32((rows, r), 0.05, 603))
        s = 32.0 / r
    dx = nf4.nf4_gemm_dx(W, dyb.to("cuda"), lora_a=None if a is None else a.to("cuda"),
                         lora_b=None if b is None else b.to("cuda"), lora_scale=s)
    torch.cuda.synchronize()
    p, am = oracle.quantize(w.reshape(-1))
    q, s2, mean = oracle.double_quant(am)
    wdeq = oracle.bf16_bits_to_f32(oracle.dequantize(p, w.size, qabsmax=q, absmax2=s2, mean=mean, out="bf16")).reshape(w.shape)
    dyf = syn.bf16_to_f32(dyb)
    af = None if a is None else syn.bf16_to_f32(a)
    bf = None if b is None else syn.bf16_to_f32(b)
    ref, _, _ = oracle.backward_ref(dyf, wdeq, lora_a=af, lora_b=bf, lora_scale=s)
    sabs = np.abs(dyf).astype(np.float64) @ np.abs(wdeq).astype(np.float64)
    if r:
        sabs += abs(s) * ((np.abs(dyf).astype(np.float64) @ np.abs(bf).astype(np.float64)) @ np.abs(af).astype(np.float64))
    check_full_product(_f64(dx), ref, sabs, terms=rows + 128, tile=DX_TILE, w_rel=LORA_SPLIT_REL if r else 0.0,
                       label="dx")


@pytest.mark.parametrize("name", ["gate", "down"])
@pytest.mark.parametrize("m", [1, 2, 4, 16])
def test_gemv_c3_every_row(name, m):
    """The Llama-8B MLP decode GEMVs on every output row at m = 1, 2, 4, 16.
    At m = 1 and 2 the streaming kernels take each level rounded to fp16 (11
    significant bits) and apply the block scale afterwards: the reference is
    the oracle's float32 dequantized weight and the per-element bound carries
    a 2^-11 relative weight term.  At m = 4 and 16 these shapes run on the
    matrix cores, which multiply by the weight rounded once to bf16 after
    scaling: the reference is the oracle's bf16 dequantized weight, with no
    weight term."""
    say("gemv C3 every row", name, "m", m)
    torch = need_gpu()
    wt = syn.c3_weight(name)
    rows, cols = wt.shape
    x = syn.c3_x(m, cols)
    W = nf4.quantize_weight(wt.to("cuda"), double_quant=True)
    y = nf4.nf4_gemv(W, x.to("cuda"))
    yf = nf4.nf4_gemv(W, x.to("cuda"), y_dtype=torch.float32)
    torch.cuda.synchronize()
    w_rel = 2.0 ** -11 if m <= 2 else 0.0
    wdeq = oracle_wdeq_full("c3:" + name, out="f32" if m <= 2 else "bf16")
    xf = syn.bf16_to_f32(x)
    ref = oracle.matmul_ref(xf, wdeq)
    sabs = _abs_product(xf, wdeq)
    check_full_product(_f64(y), ref, sabs, terms=cols, tile=GEMV_TILE, w_rel=w_rel, label="bf16 out")
    # float32 output: no final bf16 rounding, so the 2^-8 term is not needed
    gotf = yf.cpu().numpy().astype(np.float64)
    bound = (cols * 2.0 ** -24 + w_rel) * sabs + 1e-30
    assert float((np.abs(gotf - ref) / bound).max()) <= 1.0
