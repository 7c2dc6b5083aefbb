"""The 80-layer 70B-shaped stack at full size, on sampled layers: each
layer's seven weights are drawn on the device exactly as the bench's stack
leg draws them (synthetic.c5_weight_device).  Quantization and double
quantization are checked against the oracle bit for bit -- every block's
absmax, every int8 code, group scale and the mean, and the packed codes of
sampled blocks (each block quantizes on its own), every packed byte of
layer 0's 8192 x 8192 q projection -- and layer 0's decode GEMV on sampled
rows within the matmul tolerance (bitsandbytes tool page, "How it
works" and "Double quantization")."""

from __future__ import annotations

import numpy as np
import pytest

import dequant_matmul_nf4_amd as nf4
import oracle
import synthetic as syn
from tests.gpu_common import MATMUL_RTOL, need_gpu, oracle_rows_dequant_bf16, say

pytestmark = pytest.mark.gpu


def _host_f32(w_bf16):
    import torch
    return w_bf16.to(torch.float32).cpu().numpy().reshape(-1)


@pytest.mark.parametrize("layer", [0, 41, 79])
def test_c5_layer_quantize_double_quant(layer):
    torch = need_gpu()
    rng = np.random.default_rng(100 + layer)
    for name in syn.C5_ORDER:
        rows, cols = syn.C5_SHAPES[name]
        say("c5 layer", layer, name, rows, cols)
        w = syn.c5_weight_device(layer, name)
        packed, absmax = nf4.nf4_quantize(w)
        q, s2, mean = nf4.nf4_double_quant(absmax)
        torch.cuda.synchronize()
        wf = _host_f32(w)
        del w
        nb = wf.size // 64
        a_or = oracle.block_absmax(wf)
        assert np.array_equal(absmax.cpu().numpy().view(np.uint32), a_or.view(np.uint32))
        q_or, s2_or, mean_or = oracle.double_quant(a_or)
        assert np.array_equal(q.cpu().numpy(), q_or)
        assert np.array_equal(s2.cpu().numpy().view(np.uint32), s2_or.view(np.uint32))
        assert np.float32(mean.item()).view(np.uint32) == np.float32(mean_or).view(np.uint32)
        blk = np.unique(np.concatenate([[0, nb - 1], rng.choice(nb, 2048, replace=False)]))
        p_or, a_s = oracle.quantize(wf.reshape(nb, 64)[blk].reshape(-1))
        got = packed.cpu().numpy().reshape(nb, 32)[blk].reshape(-1)
        assert np.array_equal(got, p_or)
        assert np.array_equal(a_s.view(np.uint32), a_or[blk].view(np.uint32))


def test_c5_layer0_gemv_sampled_rows():
    torch = need_gpu()
    rng = np.random.default_rng(7)
    g = torch.Generator(device="cuda")
    g.manual_seed(5_000_009)
    for name in syn.C5_ORDER:
        rows, cols = syn.C5_SHAPES[name]
        say("c5 layer 0 gemv", name, rows, cols)
        w = syn.c5_weight_device(0, name)
        W = nf4.quantize_weight(w, double_quant=True)
        x = torch.randn((1, cols), generator=g, device="cuda").to(torch.bfloat16)
        y = nf4.nf4_gemv(W, x, y_dtype=torch.float32)
        torch.cuda.synchronize()
        wf = _host_f32(w).reshape(rows, cols)
        del w
        sel = np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, 128, replace=False)]))
        absmax_all = oracle.block_absmax(wf.reshape(-1))
        wdeq = oracle_rows_dequant_bf16(wf[sel], sel, cols, absmax_all, True)
        ref = oracle.matmul_ref(syn.bf16_to_f32(x), wdeq)
        got = y.cpu().numpy().astype(np.float64)[:, sel]
        e = oracle.rel_frobenius(got, ref)
        say(f"  rel err {e:.2e}")
        assert e <= MATMUL_RTOL


def test_c5_layer0_q_every_packed_byte():
    """Every packed byte of one full 70B-shaped matrix (layer 0's q
    projection, 8192 x 8192, 32 MiB of codes) against the oracle's
    quantization of the whole matrix, with its absmax and double-quantized
    scales."""
    torch = need_gpu()
    say("c5 layer 0 q: every packed byte")
    w = syn.c5_weight_device(0, "q")
    W = nf4.quantize_weight(w, double_quant=True)
    _, absmax = nf4.nf4_quantize(w)
    torch.cuda.synchronize()
    wf = _host_f32(w)
    del w
    p_or, a_or = oracle.quantize(wf)
    assert np.array_equal(W.packed.cpu().numpy(), p_or)
    assert np.array_equal(absmax.cpu().numpy().view(np.uint32), a_or.view(np.uint32))
    q_or, s2_or, mean_or = oracle.double_quant(a_or)
    assert np.array_equal(W.qabsmax.cpu().numpy(), q_or)
    assert np.array_equal(W.absmax2.cpu().numpy().view(np.uint32), s2_or.view(np.uint32))
    assert np.float32(W.mean.item()).view(np.uint32) == np.float32(mean_or).view(np.uint32)
