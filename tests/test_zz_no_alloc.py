"""nf4_double_quant_noalloc, the entry point for callers that cannot
allocate device memory, against nf4_double_quant (the entry point it is a
variant of): bit-identical codes, group scales and mean on two calls in a
row, the second on a smaller input, through the C ABI.  The second call also
checks that the static scratch's contents left by the first call do not leak
into the result, and a third call compares the first input again."""

from __future__ import annotations

import numpy as np
import pytest

import dequant_matmul_nf4_amd as nf4
import oracle
import synthetic as syn
from tests.gpu_common import need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _absmax_of(w):
    _, absmax = nf4.nf4_quantize(w)
    return absmax


def _pair(absmax):
    import torch
    nb = absmax.numel()
    dev = absmax.device
    mk = lambda: (torch.full((nb,), 99, dtype=torch.int8, device=dev),
                  torch.full(((nb + 255) // 256,), -1.0, dtype=torch.float32, device=dev),
                  torch.full((1,), -1.0, dtype=torch.float32, device=dev))
    q0, s0, m0 = mk()
    nf4.nf4_double_quant(absmax, q0, s0, m0)
    q1, s1, m1 = mk()
    nf4.nf4_double_quant_noalloc(absmax, q1, s1, m1)
    torch.cuda.synchronize()
    return (q0, s0, m0), (q1, s1, m1)


def _same(a, b):
    import torch
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.int8 else x.view(torch.int32),
                           y.view(torch.uint8) if y.dtype == torch.int8 else y.view(torch.int32))


def test_noalloc_double_quant_matches_workspace_form():
    torch = need_gpu()
    say("noalloc double quant: 4096x4096 outlier weight, then 1000 + 3 scales, then the first again")
    big = _absmax_of(syn.c2_weight().to("cuda"))            # 262144 scales: all 256 partial rows
    ref, got = _pair(big)
    _same(ref, got)
    small_w = to_dev(syn.normal_f32((1003, 64), 0.5, 77))  # 1003 scales, ragged last group
    small = _absmax_of(small_w)
    ref2, got2 = _pair(small)
    _same(ref2, got2)
    q_or, s2_or, mean_or = oracle.double_quant(small.cpu().numpy())
    assert np.array_equal(got2[0].cpu().numpy(), q_or)
    assert np.array_equal(got2[1].cpu().numpy().view(np.uint32), s2_or.view(np.uint32))
    assert np.float32(got2[2].item()).view(np.uint32) == np.float32(mean_or).view(np.uint32)
    ref3, got3 = _pair(big)
    _same(ref3, got3)
    _same(ref, got3)


def test_noalloc_rejects_bad_arguments_before_launch():
    torch = need_gpu()
    a = torch.ones(300, dtype=torch.float32, device="cuda")
    q = torch.empty(300, dtype=torch.int8, device="cuda")
    s2 = torch.empty(2, dtype=torch.float32, device="cuda")
    m = torch.empty(1, dtype=torch.float32, device="cuda")
    L = nf4.lib()
    assert L.nf4_double_quant_noalloc(a.data_ptr(), 0, 256, q.data_ptr(), s2.data_ptr(), m.data_ptr(), None) == nf4.NF4_ERR_SIZE
    assert L.nf4_double_quant_noalloc(a.data_ptr(), 1 << 31, 256, q.data_ptr(), s2.data_ptr(), m.data_ptr(), None) == nf4.NF4_ERR_SIZE
    assert L.nf4_double_quant_noalloc(a.data_ptr(), 300, 128, q.data_ptr(), s2.data_ptr(), m.data_ptr(), None) == nf4.NF4_ERR_BLOCKSIZE
    assert L.nf4_double_quant_noalloc(None, 300, 256, q.data_ptr(), s2.data_ptr(), m.data_ptr(), None) == nf4.NF4_ERR_NULL
