"""GPU parity of the FP4 code book (the E2M1 reading): nf4_quantize_fp4
bit-exact against the oracle's quantize(kind="fp4") (codes, packed bytes,
absmax) on ragged sizes, zero blocks and the 4096x4096 outlier weight;
dequantized weights and the LoRA merge bit-exact; the matmuls (GEMV at
M = 1, 2, 4, 16, GEMM with LoRA, input gradient) within the 1e-2 relative
Frobenius bound against the oracle's products on its FP4-dequantized
weights; a one-hot GEMV returns the FP4 level times the scale exactly."""

from __future__ import annotations

import numpy as np
import pytest

import dequant_matmul_nf4_amd as nf4
import oracle
import synthetic as syn
from tests.gpu_common import MATMUL_RTOL, bf16_bits, f32_bits, need_gpu, say, to_dev, u8

pytestmark = pytest.mark.gpu


def _wdeq_bf16(w_f32: np.ndarray, dq: bool = True) -> np.ndarray:
    p, a = oracle.quantize(w_f32.reshape(-1), kind="fp4")
    if dq:
        q, s2, mean = oracle.double_quant(a)
        bits = oracle.dequantize(p, w_f32.size, qabsmax=q, absmax2=s2, mean=mean, out="bf16", kind="fp4")
    else:
        bits = oracle.dequantize(p, w_f32.size, absmax=a, out="bf16", kind="fp4")
    return oracle.bf16_bits_to_f32(bits).reshape(w_f32.shape)


def _f64(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("n", [1, 63, 64, 65, 64 * 257 + 3, 64 * 1000 + 17, 4096 * 64])
@pytest.mark.parametrize("bf16", [False, True])
def test_quantize_fp4_bit_exact(n, bf16):
    say("quantize fp4", n, "bf16" if bf16 else "f32")
    torch = need_gpu()
    x = syn.random_blocks_f32(n, 1000 + n)
    if n >= 128:
        x[64:128] = 0.0  # an all-zero block
    if bf16:
        xb = syn.to_bf16(x)
        xin, xf = xb.to("cuda"), syn.bf16_to_f32(xb)
    else:
        xin, xf = to_dev(x), x
    packed, absmax = nf4.nf4_quantize(xin, fp4=True)
    torch.cuda.synchronize()
    p_o, a_o = oracle.quantize(xf, kind="fp4")
    assert np.array_equal(f32_bits(absmax), a_o.view(np.uint32))
    assert np.array_equal(u8(packed), p_o)
    codes = oracle.unpack(u8(packed), n)
    assert not np.any(codes == 8)


def test_quantize_fp4_c2_full():
    """The 4096x4096 weight with 0.1 % outliers x20: every byte and scale."""
    say("quantize fp4 C2")
    torch = need_gpu()
    inp = syn.c2_inputs()
    packed, absmax = nf4.nf4_quantize(inp["w"].to("cuda"), fp4=True)
    torch.cuda.synchronize()
    p_o, a_o = oracle.quantize(syn.bf16_to_f32(inp["w"]).reshape(-1), kind="fp4")
    assert np.array_equal(u8(packed), p_o)
    assert np.array_equal(f32_bits(absmax), a_o.view(np.uint32))


@pytest.mark.parametrize("rows,cols", [(5, 128), (300, 4096), (129, 2056)])
@pytest.mark.parametrize("dq", [False, True])
def test_dequantize_fp4_bit_exact(rows, cols, dq):
    say("dequant fp4", rows, cols, dq)
    torch = need_gpu()
    w = syn.normal_f32((rows, cols), 0.02, 1100 + rows)
    W = nf4.quantize_weight(to_dev(w), double_quant=dq, quant_type="fp4")
    d32 = nf4.nf4_dequantize(W, out_dtype=torch.float32)
    d16 = nf4.nf4_dequantize(W, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    p, a = oracle.quantize(w.reshape(-1), kind="fp4")
    if dq:
        q, s2, mean = oracle.double_quant(a)
        kw = dict(qabsmax=q, absmax2=s2, mean=mean)
    else:
        kw = dict(absmax=a)
    r32 = oracle.dequantize(p, w.size, kind="fp4", **kw)
    r16 = oracle.dequantize(p, w.size, out="bf16", kind="fp4", **kw)
    assert np.array_equal(f32_bits(d32).reshape(-1), r32.view(np.uint32))
    assert np.array_equal(bf16_bits(d16).reshape(-1), r16)


@pytest.mark.parametrize("rows,cols", [(33, 192), (1024, 4096), (300, 65 * 64 * 4)])
@pytest.mark.parametrize("m", [1, 2, 4, 16])
def test_gemv_fp4(rows, cols, m):
    say("gemv fp4", rows, cols, "m", m)
    torch = need_gpu()
    w = syn.normal_f32((rows, cols), 0.02, 1200 + rows + m)
    xb = syn.to_bf16(syn.normal_f32((m, cols), 1.0, 1201 + m))
    W = nf4.quantize_weight(to_dev(w), quant_type="fp4")
    y = nf4.nf4_gemv(W, xb.to("cuda"), y_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.matmul_ref(syn.bf16_to_f32(xb), _wdeq_bf16(w))
    e = oracle.rel_frobenius(_f64(y), ref)
    say(f"  rel err {e:.2e}")
    assert e <= MATMUL_RTOL


def test_gemv_fp4_one_hot_returns_the_scaled_level():
    """x = e_k at m = 1: y = fl32(fp16(level[code]) * a_hat) exactly (the
    decode kernel keeps each level as fp16), so a wrong code book shows at
    once."""
    say("gemv fp4 one-hot")
    torch = need_gpu()
    rows, cols = 64, 256
    w = syn.normal_f32((rows, cols), 0.02, 1210)
    W = nf4.quantize_weight(to_dev(w), quant_type="fp4")
    p, a = oracle.quantize(w.reshape(-1), kind="fp4")
    q, s2, mean = oracle.double_quant(a)
    a_hat = oracle.dequant_scales(q, s2, mean)
    codes = oracle.unpack(p, w.size).reshape(rows, cols)
    lv16 = oracle.fp4_codebook().astype(np.float16).astype(np.float32)
    for k in (0, 77, 255):
        x = torch.zeros((1, cols), dtype=torch.bfloat16, device="cuda")
        x[0, k] = 1.0
        y = nf4.nf4_gemv(W, x, y_dtype=torch.float32)
        torch.cuda.synchronize()
        blk = (np.arange(rows) * cols + k) // 64
        expect = (lv16[codes[:, k]] * a_hat[blk]).astype(np.float32)
        assert np.array_equal(y[0].cpu().numpy().view(np.uint32), expect.view(np.uint32))


@pytest.mark.parametrize("m,rows,cols,r", [(37, 200, 128, 0), (300, 520, 1024, 16), (513, 256, 320, 33)])
def test_gemm_fp4(m, rows, cols, r):
    say("gemm fp4", m, rows, cols, "r", r)
    torch = need_gpu()
    w = syn.normal_f32((rows, cols), 0.02, 1300 + m)
    xb = syn.to_bf16(syn.normal_f32((m, cols), 1.0, 1301))
    W = nf4.quantize_weight(to_dev(w), quant_type="fp4")
    a = b = None
    s = 0.0
    if r:
        a = syn.to_bf16(syn.normal_f32((r, cols), 0.02, 1302))
        b = syn.to_bf16(syn.normal_f32((rows, r), 0.02, 1303))
        s = 32.0 / r
    y = nf4.nf4_gemm(W, xb.to("cuda"), lora_a=None if a is None else a.to("cuda"),
                     lora_b=None if b is None else b.to("cuda"), lora_scale=s)
    torch.cuda.synchronize()
    ref = oracle.matmul_ref(syn.bf16_to_f32(xb), _wdeq_bf16(w), None if a is None else syn.bf16_to_f32(a),
                            None if b is None else syn.bf16_to_f32(b), s)
    e = oracle.rel_frobenius(_f64(y), ref)
    say(f"  rel err {e:.2e}")
    assert e <= MATMUL_RTOL


@pytest.mark.parametrize("m,rows,cols,r", [(37, 200, 128, 0), (300, 520, 1024, 16)])
def test_gemm_dx_fp4(m, rows, cols, r):
    say("gemm_dx fp4", m, rows, cols, "r", r)
    torch = need_gpu()
    w = syn.normal_f32((rows, cols), 0.02, 1400 + m)
    dyb = syn.to_bf16(syn.normal_f32((m, rows), 1.0, 1401))
    W = nf4.quantize_weight(to_dev(w), quant_type="fp4")
    a = b = None
    s = 0.0
    if r:
        a = syn.to_bf16(syn.normal_f32((r, cols), 0.02, 1402))
        b = syn.to_bf16(syn.normal_f32((rows, r), 0.02, 1403))
        s = 32.0 / r
    dx = nf4.nf4_gemm_dx(W, dyb.to("cuda"), lora_a=None if a is None else a.to("cuda"),
                         lora_b=None if b is None else b.to("cuda"), lora_scale=s)
    torch.cuda.synchronize()
    ref, _, _ = oracle.backward_ref(syn.bf16_to_f32(dyb), _wdeq_bf16(w),
                                    lora_a=None if a is None else syn.bf16_to_f32(a),
                                    lora_b=None if b is None else syn.bf16_to_f32(b), lora_scale=s)
    e = oracle.rel_frobenius(_f64(dx), ref)
    say(f"  rel err {e:.2e}")
    assert e <= MATMUL_RTOL


def test_lora_merge_fp4_bit_exact():
    say("merge fp4")
    torch = need_gpu()
    rows, cols, r = 129, 2056, 16
    w = syn.normal_f32((rows, cols), 0.02, 1500)
    a = syn.to_bf16(syn.normal_f32((r, cols), 0.01, 1501))
    b = syn.to_bf16(syn.normal_f32((rows, r), 0.01, 1502))
    W = nf4.quantize_weight(to_dev(w), quant_type="fp4")
    out = nf4.nf4_lora_merge(W, a.to("cuda"), b.to("cuda"), 2.0)
    torch.cuda.synchronize()
    p, am = oracle.quantize(w.reshape(-1), kind="fp4")
    q, s2, mean = oracle.double_quant(am)
    deq = oracle.dequantize(p, w.size, qabsmax=q, absmax2=s2, mean=mean, kind="fp4").reshape(rows, cols)
    ref = oracle.lora_merge(deq, syn.bf16_to_f32(a), syn.bf16_to_f32(b), 2.0, "bf16")
    assert np.array_equal(bf16_bits(out), ref.reshape(rows, cols))


def test_fp4_with_float8_second_level():
    """FP4 codes with the float8 (E4M3) second level: the two readings are
    independent, so the dequantized weights are the oracle's bit for bit and
    the GEMV stays within the bound."""
    say("fp4 + fp8 scales")
    torch = need_gpu()
    rows, cols = 257, 1024
    w = syn.normal_f32((rows, cols), 0.02, 1600)
    W = nf4.quantize_weight(to_dev(w), quant_type="fp4", dq_type="fp8")
    d16 = nf4.nf4_dequantize(W, out_dtype=torch.bfloat16)
    xb = syn.to_bf16(syn.normal_f32((1, cols), 1.0, 1601))
    y = nf4.nf4_gemv(W, xb.to("cuda"), y_dtype=torch.float32)
    torch.cuda.synchronize()
    p, a = oracle.quantize(w.reshape(-1), kind="fp4")
    q, s2, mean = oracle.double_quant_f8(a)
    r16 = oracle.dequantize(p, w.size, qabsmax=q, absmax2=s2, mean=mean, out="bf16", dq_kind="fp8", kind="fp4")
    assert np.array_equal(bf16_bits(d16).reshape(-1), r16)
    ref = oracle.matmul_ref(syn.bf16_to_f32(xb), oracle.bf16_bits_to_f32(r16).reshape(rows, cols))
    assert oracle.rel_frobenius(_f64(y), ref) <= MATMUL_RTOL


@pytest.mark.parametrize("m", [1, 4])
def test_fp4_gemv_large_sampled_rows(m):
    """A 16384x8192 FP4 weight (the streaming kernel at m = 1 and m = 4):
    all codes bit-exact, sampled output rows against the oracle."""
    say("fp4 gemv large", m)
    torch = need_gpu()
    rows, cols = 16384, 8192
    w = syn.normal_f32((rows, cols), 0.02, 1700 + m)
    x = syn.to_bf16(syn.normal_f32((m, cols), 1.0, 1701))
    W = nf4.quantize_weight(to_dev(w), quant_type="fp4")
    y = nf4.nf4_gemv(W, x.to("cuda"), y_dtype=torch.float32)
    torch.cuda.synchronize()
    p, a = oracle.quantize(w.reshape(-1), kind="fp4")
    assert np.array_equal(u8(W.packed), p)
    q, s2, mean = oracle.double_quant(a)
    a_hat = oracle.dequant_scales(q, s2, mean)
    rng = np.random.default_rng(9)
    sel = np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, 96, replace=False)]))
    codes = oracle.unpack(p, w.size).reshape(rows, cols)[sel]
    blk = (sel[:, None] * cols + np.arange(cols)[None, :]) // 64
    wdeq = (oracle.fp4_codebook()[codes] * a_hat[blk]).astype(np.float32)
    wdeq = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(wdeq)).reshape(sel.size, cols)
    ref = oracle.matmul_ref(syn.bf16_to_f32(x), wdeq)
    e = oracle.rel_frobenius(_f64(y)[:, sel], ref)
    say(f"  rel err {e:.2e}")
    assert e <= MATMUL_RTOL
