"""Calls made on a side stream, with the binding allocating the outputs and
workspaces: right after each call the default stream allocates and fills new
tensors of the same sizes (the caching allocator would hand them the memory
of any buffer the binding dropped while the side stream still uses it).  The
results must equal those of the same calls on the default stream."""

from __future__ import annotations

import pytest

import dequant_matmul_nf4_amd as nf4
import synthetic as syn
from tests.gpu_common import need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _scribble(torch, like, rounds=4):
    """New tensors of the same sizes on the current stream, filled at once."""
    keep = []
    for _ in range(rounds):
        for t in like:
            keep.append(torch.full((t.numel() * t.element_size(),), 0xA5, dtype=torch.uint8, device="cuda"))
    return keep


def test_side_stream_calls_keep_their_buffers():
    torch = need_gpu()
    rows, cols, m, r = 1536, 2048, 64, 16
    say("side stream", rows, cols, m, r)
    w = to_dev(syn.normal_f32((rows, cols), 0.02, 301)).to(torch.bfloat16)
    x1 = syn.to_bf16(syn.normal_f32((1, cols), 1.0, 302)).to("cuda")
    xm = syn.to_bf16(syn.normal_f32((m, cols), 1.0, 303)).to("cuda")
    dy = syn.to_bf16(syn.normal_f32((m, rows), 1.0, 304)).to("cuda")
    a = syn.to_bf16(syn.normal_f32((r, cols), 0.01, 305)).to("cuda")
    b = syn.to_bf16(syn.normal_f32((rows, r), 0.01, 306)).to("cuda")

    def run(stream):
        W = nf4.quantize_weight(w, double_quant=True, stream=stream)
        q, s2, mean = nf4.nf4_double_quant(W_absmax(W, stream), stream=stream)
        y1 = nf4.nf4_gemv(W, x1, stream=stream)
        y16 = nf4.nf4_gemv(W, xm[:16], stream=stream)
        yb = nf4.nf4_gemv_batched([W, W], [x1, x1], stream=stream)
        ym = nf4.nf4_gemm(W, xm, lora_a=a, lora_b=b, lora_scale=2.0, stream=stream)
        dx = nf4.nf4_gemm_dx(W, dy, lora_a=a, lora_b=b, lora_scale=2.0, stream=stream)
        da, db = nf4.nf4_lora_grads(xm, dy, a, b, 2.0, stream=stream)
        deq = nf4.nf4_dequantize(W, out_dtype=torch.bfloat16, stream=stream)
        return [W.packed, W.qabsmax, W.absmax2, W.mean, q, s2, mean, y1, y16, yb[0], yb[1], ym, dx, da, db, deq]

    def W_absmax(W, stream):
        _, am = nf4.nf4_quantize(w, stream=stream)
        return am

    ref = run(None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    got = run(side)
    junk = _scribble(torch, got)  # on the current stream, while the side stream may still run
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    for i, (g, e) in enumerate(zip(got, ref)):
        assert torch.equal(g.view(torch.uint8), e.view(torch.uint8)), i


def test_side_stream_calls_with_strided_inputs():
    """Activations whose leading dimensions do not merge (a [seq, batch,
    hidden] view of a [batch, seq, hidden] tensor): the binding's reshape to
    rows copies them into contiguous tensors of its own, which must live
    until the side stream has read them."""
    torch = need_gpu()
    rows, cols, r = 1024, 2048, 16
    seq, batch = 12, 4  # m = 48 rows; the GEMV takes the first 4 x 4
    say("side stream, non-mergeable activations", rows, cols, seq * batch, r)
    w = to_dev(syn.normal_f32((rows, cols), 0.02, 311)).to(torch.bfloat16)
    W = nf4.quantize_weight(w, double_quant=True)
    xb = syn.to_bf16(syn.normal_f32((batch * seq, cols), 1.0, 312)).to("cuda").view(batch, seq, cols)
    dyb = syn.to_bf16(syn.normal_f32((batch * seq, rows), 1.0, 313)).to("cuda").view(batch, seq, rows)
    xs, dys = xb.transpose(0, 1), dyb.transpose(0, 1)  # [seq, batch, .]
    assert xs.reshape(-1, cols).data_ptr() != xs.data_ptr()  # reshape must copy
    a = syn.to_bf16(syn.normal_f32((r, cols), 0.01, 314)).to("cuda")
    b = syn.to_bf16(syn.normal_f32((rows, r), 0.01, 315)).to("cuda")

    def run(x, dy, stream):
        y16 = nf4.nf4_gemv(W, x[:4], stream=stream)
        ym = nf4.nf4_gemm(W, x, lora_a=a, lora_b=b, lora_scale=2.0, stream=stream)
        dx = nf4.nf4_gemm_dx(W, dy, lora_a=a, lora_b=b, lora_scale=2.0, stream=stream)
        da, db = nf4.nf4_lora_grads(x, dy, a, b, 2.0, stream=stream)
        return [y16, ym, dx, da, db]

    torch.cuda.synchronize()
    ref = run(xs.contiguous(), dys.contiguous(), None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    got = run(xs, dys, side)
    junk = _scribble(torch, [xs.contiguous(), dys.contiguous()] + got)
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    for i, (g, e) in enumerate(zip(got, ref)):
        assert torch.equal(g.view(torch.uint8), e.view(torch.uint8)), i
