"""GPU parity of nf4_double_quant_batched (bitsandbytes tool page, "Double
quantization"), the double quantization of several scale arrays in one pair
of launches: every array's codes, group scales and mean bit-identical to
nf4_double_quant (int8) or nf4_double_quant_f8 (float8) on that array alone,
and, on small arrays, to the oracle's double_quant / double_quant_f8.  Sizes
cover a lone scale, tails of 1-3 scales past the last 16-byte vector, groups
of 256 with ragged ends, arrays below and above the 2^21 scales where the
single call changes workgroup size, and scales spread over a wide exponent
range (every digit of the exact sum)."""

from __future__ import annotations

import numpy as np
import pytest

import dequant_matmul_nf4_amd as nf4
import oracle
import synthetic as syn
from tests.gpu_common import need_gpu, say

pytestmark = pytest.mark.gpu


def _scales(torch, n, seed, wide=False, around=None):
    """Scales like a weight's (U(0.01, 0.06)), spread over 2^-120 .. 2^120
    (wide), or (around = k) in [2^k, 2^(k+1)), so that the group maxima of
    |a - mean| sit near 2^(k-1): k = -100 gives groups below 2^-80, where the
    quotient takes the IEEE division per value, k = -79 groups on both sides
    of 2^-80."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    if wide:
        e = torch.randint(-120, 120, (n,), generator=g, device="cuda").float()
        return (torch.rand(n, generator=g, device="cuda") + 1.0) * torch.exp2(e)
    if around is not None:
        return (torch.rand(n, generator=g, device="cuda") + 1.0) * 2.0 ** around
    return torch.rand(n, generator=g, device="cuda") * 0.05 + 0.01


def _same(a, b):
    import torch
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("fp8", [False, True], ids=["int8", "fp8"])
def test_batched_equals_single_calls(fp8):
    torch = need_gpu()
    sizes = [1, 3, 255, 257, 1000003, 131072, 4096 * 64 + 5, 2 ** 21 + 771]
    say("dq batched vs single", "fp8" if fp8 else "int8", sizes)
    arrays = [_scales(torch, n, 40 + i, wide=(i % 3 == 1)) for i, n in enumerate(sizes)]
    got = nf4.nf4_double_quant_batched(arrays, fp8=fp8)
    again = nf4.nf4_double_quant_batched(arrays, fp8=fp8)
    single = [nf4.nf4_double_quant(a, fp8=fp8) for a in arrays]
    torch.cuda.synchronize()
    for i, (g1, g2, s1) in enumerate(zip(got, again, single)):
        for k, (x, y, z) in enumerate(zip(g1, g2, s1)):
            assert _same(x, z), (sizes[i], k)
            assert _same(x, y), (sizes[i], k, "not deterministic")


@pytest.mark.parametrize("fp8", [False, True], ids=["int8", "fp8"])
def test_batched_small_arrays_bit_exact_against_oracle(fp8):
    torch = need_gpu()
    sizes = [1, 2, 7, 256, 513, 5000, 3000, 3000, 3000, 777]
    around = [None] * 6 + [-100, -79, -78, 100]
    say("dq batched vs oracle", sizes)
    arrays = [_scales(torch, n, 70 + i, wide=(i % 2 == 0 and around[i] is None), around=around[i])
              for i, n in enumerate(sizes)]
    got = nf4.nf4_double_quant_batched(arrays[:8], fp8=fp8) + nf4.nf4_double_quant_batched(arrays[8:], fp8=fp8)
    single = [nf4.nf4_double_quant(a, fp8=fp8) for a in arrays]
    torch.cuda.synchronize()
    for g1, s1 in zip(got, single):
        for x, y in zip(g1, s1):
            assert _same(x, y)
    for a, (q, s2, mu) in zip(arrays, got):
        a_np = a.cpu().numpy()
        oq, os2, omu = (oracle.double_quant_f8 if fp8 else oracle.double_quant)(a_np)
        assert np.array_equal(q.cpu().numpy().view(np.uint8), np.asarray(oq).view(np.uint8))
        assert np.array_equal(s2.cpu().numpy().view(np.uint32), np.asarray(os2, np.float32).view(np.uint32))
        assert np.array_equal(mu.cpu().numpy().view(np.uint32), np.asarray([omu], np.float32).view(np.uint32))


def test_batched_single_array_and_caller_outputs():
    """count = 1, and outputs given by the caller (the binding allocates nothing)."""
    torch = need_gpu()
    say("dq batched count 1")
    a = _scales(torch, 3670016, 90)
    outs = [(torch.empty(a.numel(), dtype=torch.int8, device="cuda"),
             torch.empty((a.numel() + 255) // 256, dtype=torch.float32, device="cuda"),
             torch.empty(1, dtype=torch.float32, device="cuda"))]
    ws = torch.empty(nf4.lib().nf4_double_quant_batched_workspace(1), dtype=torch.uint8, device="cuda")
    got = nf4.nf4_double_quant_batched([a], outs=outs, workspace=ws)
    ref = nf4.nf4_double_quant(a)
    torch.cuda.synchronize()
    assert got[0][0] is outs[0][0]
    for x, y in zip(got[0], ref):
        assert _same(x, y)


def test_batched_70b_layer_scales():
    """The seven weights of a 70B-shaped layer (drawn as the benchmark draws
    them), quantized one by one, then their scales double-quantized in one
    call: identical to seven single calls."""
    torch = need_gpu()
    say("dq batched 70B layer")
    absmaxes = []
    for name in syn.C5_ORDER:
        w = syn.c5_weight_device(3, name)
        _, am = nf4.nf4_quantize(w)
        absmaxes.append(am)
        del w
    got = nf4.nf4_double_quant_batched(absmaxes)
    single = [nf4.nf4_double_quant(a) for a in absmaxes]
    torch.cuda.synchronize()
    for name, g1, s1 in zip(syn.C5_ORDER, got, single):
        for x, y in zip(g1, s1):
            assert _same(x, y), name
