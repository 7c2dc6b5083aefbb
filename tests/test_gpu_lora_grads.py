"""GPU parity of nf4_lora_grads (dA = s (dY B)^T X, dB = s dY^T (X A^T),
float32) against the oracle's float64 backward_ref: relative Frobenius error
<= 1e-2 (MATMUL_RTOL), at small ragged shapes and at the full C4 size."""

from __future__ import annotations

import numpy as np
import pytest

import dequant_matmul_nf4_amd as nf4
import oracle
import synthetic as syn
from tests.gpu_common import MATMUL_RTOL, need_gpu, say

pytestmark = pytest.mark.gpu


def _ref(x, dy, a, b, s):
    rows, cols = b.shape[0], a.shape[1]
    _, da, db = oracle.backward_ref(syn.bf16_to_f32(dy), np.zeros((rows, cols)), x=syn.bf16_to_f32(x),
                                    lora_a=syn.bf16_to_f32(a), lora_b=syn.bf16_to_f32(b), lora_scale=s)
    return da, db


# m below one wave's share, ragged splits, columns that are not a multiple of
# a workgroup's 512, ranks across the 16-entry passes
@pytest.mark.parametrize("m,rows,cols,r", [(1, 8, 8, 1), (3, 64, 136, 16), (37, 200, 520, 16), (300, 1032, 264, 33),
                                           (1000, 512, 1024, 64), (4099, 96, 72, 7)])
def test_lora_grads_small(m, rows, cols, r):
    say("lora_grads", m, rows, cols, "r", r)
    torch = need_gpu()
    seed = m + rows + r
    x = syn.to_bf16(syn.normal_f32((m, cols), 1.0, seed))
    dy = syn.to_bf16(syn.normal_f32((m, rows), 1.0, seed + 1))
    a = syn.to_bf16(syn.normal_f32((r, cols), 0.02, seed + 2))
    b = syn.to_bf16(syn.normal_f32((rows, r), 0.02, seed + 3))
    s = 32.0 / r
    da, db = nf4.nf4_lora_grads(x.cuda(), dy.cuda(), a.cuda(), b.cuda(), s)
    torch.cuda.synchronize()
    rda, rdb = _ref(x, dy, a, b, s)
    ea = oracle.rel_frobenius(da.cpu().numpy(), rda)
    eb = oracle.rel_frobenius(db.cpu().numpy(), rdb)
    say(f"  rel err dA {ea:.2e} dB {eb:.2e}")
    assert ea <= MATMUL_RTOL and eb <= MATMUL_RTOL


def test_lora_grads_one_of_two_and_closed_forms():
    """Asking for one gradient gives the same values as asking for both; with
    B = 0 dA is exactly zero; a one-hot dY row and x row give dB = s A^T at
    one entry."""
    say("lora_grads closed forms")
    torch = need_gpu()
    m, rows, cols, r = 64, 136, 264, 16
    x = syn.to_bf16(syn.normal_f32((m, cols), 1.0, 51)).cuda()
    dy = syn.to_bf16(syn.normal_f32((m, rows), 1.0, 52)).cuda()
    a = syn.to_bf16(syn.normal_f32((r, cols), 0.02, 53)).cuda()
    b = syn.to_bf16(syn.normal_f32((rows, r), 0.02, 54)).cuda()
    da, db = nf4.nf4_lora_grads(x, dy, a, b, 2.0)
    da1, _ = nf4.nf4_lora_grads(x, dy, a, b, 2.0, want=("da",))
    _, db1 = nf4.nf4_lora_grads(x, dy, a, b, 2.0, da=None, want=("db",))
    nf4.nf4_lora_grads(x, dy, a, b, 2.0, da=torch.empty((r, cols), device="cuda"), want=())
    da0, _ = nf4.nf4_lora_grads(x, dy, a, torch.zeros_like(b), 2.0)
    torch.cuda.synchronize()
    assert torch.equal(da, da1) and torch.equal(db, db1)
    assert torch.count_nonzero(da0).item() == 0
    # one-hot: dy = e_3 (row 0), x = e_5 (row 0) and zero elsewhere -> dB[3][j] = s A[j][5]
    e_dy = torch.zeros((m, rows), dtype=torch.bfloat16, device="cuda")
    e_x = torch.zeros((m, cols), dtype=torch.bfloat16, device="cuda")
    e_dy[0, 3] = 1.0
    e_x[0, 5] = 1.0
    _, dbe = nf4.nf4_lora_grads(e_x, e_dy, a, b, 2.0)
    torch.cuda.synchronize()
    want = torch.zeros((rows, r), device="cuda")
    want[3] = 2.0 * a[:, 5].float()
    assert torch.equal(dbe, want)


def test_lora_grads_c4_full():
    """C4's adapter gradients at full size (X [4096, 4096], dY [4096, 14336],
    r = 16, alpha = 32), every element against the oracle; then rerun for
    bit-identical results."""
    say("lora_grads C4 full size")
    torch = need_gpu()
    inp = syn.c4_inputs()
    dy = syn.c4_grad()
    x, a, b = inp["x"], inp["a"], inp["b"]
    s = inp["alpha"] / inp["r"]
    xd, dyd, ad, bd = x.cuda(), dy.cuda(), a.cuda(), b.cuda()
    da, db = nf4.nf4_lora_grads(xd, dyd, ad, bd, s)
    torch.cuda.synchronize()
    rda, rdb = _ref(x, dy, a, b, s)
    ea = oracle.rel_frobenius(da.cpu().numpy(), rda)
    eb = oracle.rel_frobenius(db.cpu().numpy(), rdb)
    say(f"  rel err dA {ea:.2e} dB {eb:.2e}")
    assert ea <= MATMUL_RTOL and eb <= MATMUL_RTOL
    da2, db2 = nf4.nf4_lora_grads(xd, dyd, ad, bd, s)
    torch.cuda.synchronize()
    assert torch.equal(da, da2) and torch.equal(db, db2)
