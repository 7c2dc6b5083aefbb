"""GPU parity of nf4_quantize_batched (bitsandbytes tool page, "How it
works", Steps 1-4), the blockwise quantization of several tensors in one
launch: every tensor's packed codes and absmax bit-identical to nf4_quantize
(or nf4_quantize_fp4) on that tensor alone, for bf16 and float32 inputs;
small tensors also against the oracle; and the seven weights of a 70B-shaped
layer quantized and double-quantized with the two batched calls, identical
to quantize_weight on each."""

from __future__ import annotations

import numpy as np
import pytest

import dequant_matmul_nf4_amd as nf4
import oracle
import synthetic as syn
from tests.gpu_common import need_gpu, say


pytestmark = pytest.mark.gpu


def _x(torch, n, seed, dt):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn(n, generator=g, device="cuda") * 0.02
    x[::997] *= 20.0  # outliers
    return x.to(dt)


@pytest.mark.parametrize("fp4", [False, True], ids=["nf4", "fp4"])
@pytest.mark.parametrize("bf16", [True, False], ids=["bf16", "f32"])
def test_batched_equals_single_calls(bf16, fp4):
    torch = need_gpu()
    dt = torch.bfloat16 if bf16 else torch.float32
    sizes = [1, 63, 64, 65, 1000, 64 * 1000 + 17, 4096 * 4096, 8192 * 1024]
    say("quantize batched", "bf16" if bf16 else "f32", "fp4" if fp4 else "nf4", sizes)
    xs = [_x(torch, n, 10 + i, dt) for i, n in enumerate(sizes)]
    got = nf4.nf4_quantize_batched(xs, fp4=fp4)
    single = [nf4.nf4_quantize(x, fp4=fp4) for x in xs]
    torch.cuda.synchronize()
    for n, (p1, a1), (p2, a2) in zip(sizes, got, single):
        assert torch.equal(p1, p2), n
        assert torch.equal(a1.view(torch.int32), a2.view(torch.int32)), n


@pytest.mark.parametrize("fp4", [False, True], ids=["nf4", "fp4"])
def test_batched_small_tensors_against_oracle(fp4):
    torch = need_gpu()
    sizes = [1, 7, 64, 129, 5000]
    say("quantize batched vs oracle", sizes)
    xs = [_x(torch, n, 30 + i, torch.float32) for i, n in enumerate(sizes)]
    got = nf4.nf4_quantize_batched(xs, fp4=fp4)
    torch.cuda.synchronize()
    for x, (p, a) in zip(xs, got):
        p_ref, a_ref = oracle.quantize(x.cpu().numpy(), kind="fp4" if fp4 else "nf4")
        assert np.array_equal(p.cpu().numpy(), p_ref)
        assert np.array_equal(a.cpu().numpy().view(np.uint32), a_ref.view(np.uint32))


def test_batched_70b_layer_weights():
    """A 70B-shaped layer (drawn as the benchmark draws it) through the two
    batched calls, against quantize_weight on each matrix."""
    torch = need_gpu()
    say("quantize + double quant batched, 70B layer")
    ws = [syn.c5_weight_device(7, name) for name in syn.C5_ORDER]
    got = nf4.nf4_quantize_batched(ws)
    dq = nf4.nf4_double_quant_batched([a for _, a in got])
    torch.cuda.synchronize()
    for name, w, (p, _), (q, s2, mu) in zip(syn.C5_ORDER, ws, got, dq):
        W = nf4.quantize_weight(w, double_quant=True)
        torch.cuda.synchronize()
        assert torch.equal(p, W.packed), name
        assert torch.equal(q, W.qabsmax), name
        assert torch.equal(s2.view(torch.int32), W.absmax2.view(torch.int32)), name
        assert torch.equal(mu.view(torch.int32), W.mean.view(torch.int32)), name


@pytest.mark.parametrize("qt,dq", [("nf4", "int8"), ("fp4", "fp8"), ("nf4", None)])
def test_quantize_weights_matches_quantize_weight(qt, dq):
    """The binding's quantize_weights (the two batched calls) against
    quantize_weight on each of three weights of different shapes."""
    torch = need_gpu()
    say("quantize_weights", qt, dq)
    shapes = [(300, 1024), (64, 64), (1024, 4160)]
    ws = [_x(torch, r * c, 50 + i, torch.bfloat16).reshape(r, c) for i, (r, c) in enumerate(shapes)]
    got = nf4.quantize_weights(ws, double_quant=dq is not None, dq_type=dq or "int8", quant_type=qt)
    ref = [nf4.quantize_weight(w, double_quant=dq is not None, dq_type=dq or "int8", quant_type=qt) for w in ws]
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert (a.rows, a.cols, a.dq_type, a.quant_type) == (b.rows, b.cols, b.dq_type, b.quant_type)
        assert torch.equal(a.packed, b.packed)
        for f in ("absmax", "qabsmax", "absmax2", "mean"):
            x, y = getattr(a, f), getattr(b, f)
            assert (x is None) == (y is None), f
            if x is not None:
                assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f

