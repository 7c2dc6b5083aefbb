"""LoRA merge (tutorial page, "Merging LoRA Adapters After Fine-Tuning"):
W' = round(deq(W) + s * B . A) into bf16 or fp16, bit for bit against the
oracle, through the C ABI."""

from __future__ import annotations

import numpy as np
import pytest

import dequant_matmul_nf4_amd as nf4
import oracle
import synthetic as syn
from tests.gpu_common import need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _oracle_deq(w_f32: np.ndarray, dq: bool) -> np.ndarray:
    p, a = oracle.quantize(w_f32.reshape(-1))
    if dq:
        q, s2, mean = oracle.double_quant(a)
        return oracle.dequantize(p, w_f32.size, qabsmax=q, absmax2=s2, mean=mean, out="f32").reshape(w_f32.shape)
    return oracle.dequantize(p, w_f32.size, absmax=a, out="f32").reshape(w_f32.shape)


@pytest.mark.parametrize("rows,cols,r", [(1, 8, 1), (7, 64, 16), (33, 200, 5), (300, 4096, 16), (129, 2056, 64)])
@pytest.mark.parametrize("dq", [True, False])
@pytest.mark.parametrize("out", ["bf16", "f16"])
def test_merge_bit_exact(rows, cols, r, dq, out):
    torch = need_gpu()
    say("merge", rows, cols, r, "dq" if dq else "plain", out)
    w = syn.normal_f32((rows, cols), 0.02, rows + 3 * cols + r)
    a = syn.to_bf16(syn.normal_f32((r, cols), 0.01, 31 + r))
    b = syn.to_bf16(syn.normal_f32((rows, r), 0.01, 32 + r))
    s = 32.0 / r
    W = nf4.quantize_weight(to_dev(w), double_quant=dq)
    got = nf4.nf4_lora_merge(W, a.to("cuda"), b.to("cuda"), s,
                             out_dtype=torch.bfloat16 if out == "bf16" else torch.float16)
    torch.cuda.synchronize()
    ref = oracle.lora_merge(_oracle_deq(w, dq), syn.bf16_to_f32(a), syn.bf16_to_f32(b), s, out)
    assert np.array_equal(_bits(got), ref)


def test_merge_with_zero_b_is_the_dequantized_base():
    torch = need_gpu()
    rows, cols, r = 64, 512, 16
    w = syn.normal_f32((rows, cols), 0.02, 41)
    W = nf4.quantize_weight(to_dev(w), double_quant=True)
    a = syn.to_bf16(syn.normal_f32((r, cols), 0.01, 42)).to("cuda")
    b = torch.zeros((rows, r), dtype=torch.bfloat16, device="cuda")
    merged = nf4.nf4_lora_merge(W, a, b, 2.0)
    deq = nf4.nf4_dequantize(W, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(merged.view(torch.int16), deq.view(torch.int16))


def test_merge_c4_full_size_sampled_rows():
    """The QLoRA shape of the forward GEMM (W 14336 x 4096, r = 16, alpha = 32):
    every row the oracle checks is bit-exact."""
    torch = need_gpu()
    inp = syn.c4_inputs()
    wt = inp["w"]
    rows, cols = wt.shape
    r = inp["r"]
    s = inp["alpha"] / r
    W = nf4.quantize_weight(wt.to("cuda"), double_quant=True)
    got = nf4.nf4_lora_merge(W, inp["a"].to("cuda"), inp["b"].to("cuda"), s)
    torch.cuda.synchronize()
    w_f32 = syn.bf16_to_f32(wt)
    rng = np.random.default_rng(8)
    sel = np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, 64, replace=False)]))
    absmax_all = oracle.block_absmax(w_f32.reshape(-1))
    q, s2, mean = oracle.double_quant(absmax_all)
    a_hat = oracle.dequant_scales(q, s2, mean)
    bpr = cols // 64
    deq = np.empty((len(sel), cols), dtype=np.float32)
    for i, n in enumerate(sel):
        p, _ = oracle.quantize(w_f32[n])
        deq[i] = oracle.dequantize(p, cols, absmax=a_hat[n * bpr:(n + 1) * bpr], out="f32")
    ref = oracle.lora_merge(deq, syn.bf16_to_f32(inp["a"]), syn.bf16_to_f32(inp["b"])[sel], s, "bf16")
    assert np.array_equal(_bits(got)[sel], ref)
