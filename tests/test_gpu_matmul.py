"""GPU parity of nf4_gemv and nf4_gemm against the oracle's float64 product of
its bf16-dequantized weights: relative Frobenius error <= 1e-2 (MATMUL_RTOL);
the GEMMs also per 128 x 256 output block (the half-tile work unit) and per
element (gpu_common.check_full_product).  The full-size workloads are checked
on every output in test_gpu_full_size.py."""

from __future__ import annotations

import numpy as np
import pytest

import dequant_matmul_nf4_amd as nf4
import oracle
import synthetic as syn
from tests.gpu_common import MATMUL_RTOL, check_full_product, need_gpu, oracle_rows_dequant_bf16, say, to_dev

pytestmark = pytest.mark.gpu


def _full_oracle_wdeq(w_f32: np.ndarray, dq: bool) -> np.ndarray:
    p, a = oracle.quantize(w_f32.reshape(-1))
    if dq:
        q, s2, mean = oracle.double_quant(a)
        bits = oracle.dequantize(p, w_f32.size, qabsmax=q, absmax2=s2, mean=mean, out="bf16")
    else:
        bits = oracle.dequantize(p, w_f32.size, absmax=a, out="bf16")
    return oracle.bf16_bits_to_f32(bits).reshape(w_f32.shape)


def _y_f64(y):
    import torch
    return y.detach().to(torch.float32).cpu().numpy().astype(np.float64)


GEMM_UNIT = (128, 256)        # half-tile work unit of nf4_gemm (rows of x, rows of W)
LORA_SPLIT_REL = 2.0 ** -16   # s T carried as two bf16 parts


def _check_gemm(y, xb, wdeq, a=None, b=None, s=0.0, label="gemm"):
    """Whole-output, per-block and per-element bounds against the oracle."""
    xf = syn.bf16_to_f32(xb)
    af = None if a is None else syn.bf16_to_f32(a)
    bf = None if b is None else syn.bf16_to_f32(b)
    ref = oracle.matmul_ref(xf, wdeq, af, bf, s)
    sabs = np.abs(xf).astype(np.float64) @ np.abs(wdeq).astype(np.float64).T
    if af is not None:
        t = np.abs(xf).astype(np.float64) @ np.abs(af).astype(np.float64).T
        sabs += abs(s) * (t @ np.abs(bf).astype(np.float64).T)
    check_full_product(_y_f64(y), ref, sabs, terms=xf.shape[1] + 128, tile=GEMM_UNIT,
                       w_rel=0.0 if a is None else LORA_SPLIT_REL, label=label)


@pytest.mark.parametrize("rows,cols", [(1, 64), (5, 128), (33, 192), (1024, 1024), (300, 4096)])
@pytest.mark.parametrize("m", [1, 2, 4, 5, 16])
@pytest.mark.parametrize("dq", [False, True])
def test_gemv_small(rows, cols, m, dq):
    say("gemv", rows, cols, "m", m, "dq" if dq else "plain")
    torch = need_gpu()
    w = syn.normal_f32((rows, cols), 0.02, rows + 7 * cols)
    xb = syn.to_bf16(syn.normal_f32((m, cols), 1.0, 99 + m))
    W = nf4.quantize_weight(to_dev(w), double_quant=dq)
    y32 = nf4.nf4_gemv(W, xb.to("cuda"), y_dtype=torch.float32)
    yb = nf4.nf4_gemv(W, xb.to("cuda"), y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.matmul_ref(syn.bf16_to_f32(xb), _full_oracle_wdeq(w, dq))
    e32 = oracle.rel_frobenius(_y_f64(y32), ref)
    eb = oracle.rel_frobenius(_y_f64(yb), ref)
    say(f"  rel err f32 {e32:.2e} bf16 {eb:.2e}")
    assert e32 <= MATMUL_RTOL and eb <= MATMUL_RTOL


def test_gemv_c1_full():
    say("gemv C1")
    torch = need_gpu()
    inp = syn.c1_inputs()
    W = nf4.quantize_weight(to_dev(inp["w_f32"]), double_quant=False)
    y = nf4.nf4_gemv(W, inp["x"].to("cuda"), y_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.matmul_ref(syn.bf16_to_f32(inp["x"]), _full_oracle_wdeq(inp["w_f32"], False))
    e = oracle.rel_frobenius(_y_f64(y), ref)
    say(f"  rel err {e:.2e}")
    assert e <= MATMUL_RTOL


def test_gemv_c2_full():
    say("gemv C2 4096x4096 dq")
    torch = need_gpu()
    inp = syn.c2_inputs()
    W = nf4.quantize_weight(inp["w"].to("cuda"), double_quant=True)
    y = nf4.nf4_gemv(W, inp["x"].to("cuda"))
    torch.cuda.synchronize()
    ref = oracle.matmul_ref(syn.bf16_to_f32(inp["x"]), _full_oracle_wdeq(syn.bf16_to_f32(inp["w"]), True))
    e = oracle.rel_frobenius(_y_f64(y), ref)
    say(f"  rel err {e:.2e}")
    assert e <= MATMUL_RTOL


@pytest.mark.parametrize("m", [3, 4])
def test_gemv_skinny_streaming_path_large(m):
    """m <= 4 on a matrix of at least 2^27 weights takes the streaming kernel
    with the x rows sharing each lookup: sampled rows against the oracle, and
    the result does not depend on the scale array's alignment."""
    say("gemv skinny streaming path", m)
    torch = need_gpu()
    rows, cols = 16384, 8192
    w = syn.normal_f32((rows, cols), 0.02, 31 + m)
    x = syn.to_bf16(syn.normal_f32((m, cols), 1.0, 32))
    W = nf4.quantize_weight(to_dev(w), double_quant=True)
    y = nf4.nf4_gemv(W, x.to("cuda"), y_dtype=torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    sel = np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, 128, replace=False)]))
    absmax_all = oracle.block_absmax(w.reshape(-1))
    wdeq = oracle_rows_dequant_bf16(w[sel], sel, cols, absmax_all, True)
    ref = oracle.matmul_ref(syn.bf16_to_f32(x), wdeq)
    e = oracle.rel_frobenius(_y_f64(y)[:, sel], ref)
    say(f"  rel err {e:.2e}")
    assert e <= MATMUL_RTOL


def test_gemv_one_hot_and_determinism():
    """x = e_k returns column k of the dequantized weight in closed form.  For
    m = 1 the decode GEMV takes each level rounded to fp16 and x exactly
    (scaled by a power of two that it undoes), so y[n] is exactly
    fl32(fp16(level[code]) * a_hat): the level and a_hat come from the oracle
    and the fp16 rounding (nearest even) from numpy.  That is within 2^-11 of
    the float32 dequantized value.  Two runs give identical bits."""
    say("gemv one-hot")
    torch = need_gpu()
    rows, cols = 256, 512
    w = syn.normal_f32((rows, cols), 0.02, 4)
    W = nf4.quantize_weight(to_dev(w), double_quant=True)
    p, a = oracle.quantize(w.reshape(-1))
    q, s2, mean = oracle.double_quant(a)
    a_hat = oracle.dequant_scales(q, s2, mean)
    codes = oracle.unpack(p, w.size).reshape(rows, cols)
    lv16 = oracle.codebook().astype(np.float16).astype(np.float32)
    wdeq_f32 = nf4.nf4_dequantize(W, out_dtype=torch.float32)
    for k in (0, 77, 511):
        x = torch.zeros((1, cols), dtype=torch.bfloat16, device="cuda")
        x[0, k] = 1.0
        y = nf4.nf4_gemv(W, x, y_dtype=torch.float32)
        torch.cuda.synchronize()
        blk = (np.arange(rows) * cols + k) // 64
        expect = (lv16[codes[:, k]] * a_hat[blk]).astype(np.float32)
        got = y[0].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), expect.view(np.uint32)), k
        ref = wdeq_f32[:, k]
        assert bool(((y[0] - ref).abs() <= ref.abs() * (2.0 ** -11 + 2.0 ** -22)).all())
    x = syn.to_bf16(syn.normal_f32((4, cols), 1.0, 8)).to("cuda")
    for m in (1, 4):
        y1 = nf4.nf4_gemv(W, x[:m])
        y2 = nf4.nf4_gemv(W, x[:m])
        torch.cuda.synchronize()
        assert torch.equal(y1, y2)


@pytest.mark.parametrize("m", [4, 16])
@pytest.mark.parametrize("dq", [True, False])
def test_gemv_skinny_scale_load_forms(m, dq):
    """The skinny (2 <= m <= 16) kernel reads a segment's four scale inputs
    with one aligned load when the scale array allows it, and block by block
    otherwise; both forms compute the same a_hat, so the outputs must be
    bit-identical.  Scale arrays placed at an unaligned offset force the
    block-by-block form.  Both are also checked against the oracle."""
    torch = need_gpu()
    rows, cols = 300, 4096
    say("gemv skinny scale load forms", rows, cols, m, dq)
    w = syn.normal_f32((rows, cols), 0.02, 21)
    W = nf4.quantize_weight(to_dev(w), double_quant=dq)
    x = syn.to_bf16(syn.normal_f32((m, cols), 1.0, 22)).to("cuda")
    if dq:
        buf = torch.zeros(W.qabsmax.numel() + 1, dtype=torch.int8, device="cuda")
        buf[1:].copy_(W.qabsmax)
        Wu = nf4.NF4Weight(W.packed, rows, cols, qabsmax=buf[1:], absmax2=W.absmax2, mean=W.mean)
        assert Wu.qabsmax.data_ptr() % 4 == 1
    else:
        buf = torch.zeros(W.absmax.numel() + 1, dtype=torch.float32, device="cuda")
        buf[1:].copy_(W.absmax)
        Wu = nf4.NF4Weight(W.packed, rows, cols, absmax=buf[1:])
        assert Wu.absmax.data_ptr() % 16 == 4
    ya = nf4.nf4_gemv(W, x, y_dtype=torch.float32)
    yu = nf4.nf4_gemv(Wu, x, y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(ya, yu)
    ref = oracle.matmul_ref(syn.bf16_to_f32(x), _full_oracle_wdeq(w, dq))
    err = oracle.rel_frobenius(_y_f64(ya), ref)
    assert err <= MATMUL_RTOL, err


def _oracle_wdeq_kind(w_f32: np.ndarray, dq, kind: str) -> np.ndarray:
    """The oracle's bf16 dequantized weight (as float32) for a second-level
    reading dq (None, "int8" or "fp8") and a code book kind ("nf4", "fp4")."""
    p, a = oracle.quantize(w_f32.reshape(-1), kind=kind)
    if dq is None:
        bits = oracle.dequantize(p, w_f32.size, absmax=a, out="bf16", kind=kind)
    else:
        q, s2, mean = oracle.double_quant_f8(a) if dq == "fp8" else oracle.double_quant(a)
        bits = oracle.dequantize(p, w_f32.size, qabsmax=q, absmax2=s2, mean=mean, out="bf16", dq_kind=dq, kind=kind)
    return oracle.bf16_bits_to_f32(bits).reshape(w_f32.shape)


@pytest.mark.parametrize("rows,cols,m,dq,kind", [
    (16, 64, 16, "int8", "nf4"),      # one group, one block: a segment of 1 block
    (33, 192, 7, "fp8", "fp4"),       # a segment of 3 blocks, ragged last group
    (777, 1088, 16, None, "nf4"),     # 17 blocks a row: block-by-block scale loads
    (1000, 4160, 5, "int8", "nf4"),   # 65 blocks a row, ragged rows
    (520, 4096, 8, None, "fp4"),      # plain absmax, one 16-byte load per segment
    (1040, 4096, 12, "int8", "fp4"),
    (2064, 2048, 16, "fp8", "nf4"),
    # rows wider than 64 segments of 4 blocks: tiles per (row group, wave),
    # summed over each wave's segments
    (40, 16448, 7, None, "fp4"),
    (33, 20480, 5, "fp8", "nf4"),
    (520, 24576, 16, "int8", "nf4"),
])
def test_gemv_skinny_matrix_cores_every_output(rows, cols, m, dq, kind):
    """For 5 <= m <= 16 the product runs on the matrix cores with the weight
    rounded once to bf16 after scaling, bf16(fl32(level * a_hat)), as the GEMM
    expands it (so that an MFMA may span two blocks).  Every output is checked
    against the oracle's float64 product with its bf16 dequantized weight, with
    no weight term in the per-element bound: only the float32 sums and the
    output rounding."""
    say("gemv skinny matrix cores", rows, cols, "m", m, dq, kind)
    torch = need_gpu()
    w = syn.normal_f32((rows, cols), 0.02, 17 * rows + cols)
    xb = syn.to_bf16(syn.normal_f32((m, cols), 1.0, 5 + m))
    W = nf4.quantize_weight(to_dev(w), double_quant=dq is not None, dq_type=dq or "int8", quant_type=kind)
    y32 = nf4.nf4_gemv(W, xb.to("cuda"), y_dtype=torch.float32)
    yb = nf4.nf4_gemv(W, xb.to("cuda"))
    torch.cuda.synchronize()
    wdeq = _oracle_wdeq_kind(w, dq, kind)
    xf = syn.bf16_to_f32(xb)
    ref = oracle.matmul_ref(xf, wdeq)
    sabs = np.abs(xf).astype(np.float64) @ np.abs(wdeq).astype(np.float64).T
    check_full_product(_y_f64(yb), ref, sabs, terms=cols, tile=(16, 16), label="bf16 out")
    bound = cols * 2.0 ** -24 * sabs + 1e-30
    assert float((np.abs(_y_f64(y32) - ref) / bound).max()) <= 1.0


@pytest.mark.parametrize("m", [8, 16])
def test_gemv_skinny_wide_rows_several_groups(m):
    """8192 x 16448 (65 segments of 4 blocks a row) on the matrix cores: the
    kernel keeps a tile per (row group, wave) and a workgroup takes two row
    groups.  Sampled rows (the first, the last and 128 random ones) against
    the oracle's bf16 dequantized weight, with no weight term in the bound."""
    say("gemv skinny wide rows", m)
    torch = need_gpu()
    rows, cols = 8192, 16448
    w = syn.normal_f32((rows, cols), 0.02, 41 + m)
    x = syn.to_bf16(syn.normal_f32((m, cols), 1.0, 42))
    W = nf4.quantize_weight(to_dev(w), double_quant=True)
    y = nf4.nf4_gemv(W, x.to("cuda"), y_dtype=torch.float32)
    yb = nf4.nf4_gemv(W, x.to("cuda"))
    torch.cuda.synchronize()
    rng = np.random.default_rng(43)
    sel = np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, 128, replace=False)]))
    absmax_all = oracle.block_absmax(w.reshape(-1))
    wdeq = oracle_rows_dequant_bf16(w[sel], sel, cols, absmax_all, True)
    xf = syn.bf16_to_f32(x)
    ref = oracle.matmul_ref(xf, wdeq)
    sabs = np.abs(xf).astype(np.float64) @ np.abs(wdeq).astype(np.float64).T
    check_full_product(_y_f64(yb)[:, sel], ref, sabs, terms=cols, tile=(16, 16), label="bf16 out")
    bound = cols * 2.0 ** -24 * sabs + 1e-30
    assert float((np.abs(_y_f64(y)[:, sel] - ref) / bound).max()) <= 1.0


def test_gemv_x_dynamic_range():
    """x spanning 2^-60 .. 2^60 within and across blocks, and an all-zero
    block: the per-block power-of-two scaling of x keeps the decode GEMV
    within tolerance and finite."""
    say("gemv x dynamic range")
    torch = need_gpu()
    rows, cols = 512, 1024
    w = syn.normal_f32((rows, cols), 0.02, 64)
    rng = np.random.default_rng(65)
    xf = (rng.standard_normal((1, cols)) * np.exp2(rng.integers(-60, 61, (1, cols)))).astype(np.float32)
    xf[0, 128:192] = 0.0
    xf[0, 256:320] *= np.float32(2.0 ** -60)
    xb = syn.to_bf16(xf)
    W = nf4.quantize_weight(to_dev(w), double_quant=True)
    y = nf4.nf4_gemv(W, xb.to("cuda"), y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    ref = oracle.matmul_ref(syn.bf16_to_f32(xb), _full_oracle_wdeq(w, True))
    e = oracle.rel_frobenius(_y_f64(y), ref)
    say(f"  rel err {e:.2e}")
    assert e <= MATMUL_RTOL


@pytest.mark.parametrize("rows,cols,m", [(7, 65600, 1), (40, 131072, 1), (9, 32832, 3), (20, 40960, 16)])
def test_gemv_wider_than_16_segments(rows, cols, m):
    """Rows longer than 16 x 64 blocks at m = 1 take the per-row-group kernel;
    at m > 1 these shapes run on the matrix cores with a tile per (row group,
    wave)."""
    say("gemv wide", rows, cols, "m", m)
    torch = need_gpu()
    w = syn.normal_f32((rows, cols), 0.02, 61)
    xb = syn.to_bf16(syn.normal_f32((m, cols), 1.0, 62))
    W = nf4.quantize_weight(to_dev(w), double_quant=True)
    y = nf4.nf4_gemv(W, xb.to("cuda"), y_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.matmul_ref(syn.bf16_to_f32(xb), _full_oracle_wdeq(w, True))
    e = oracle.rel_frobenius(_y_f64(y), ref)
    say(f"  rel err {e:.2e}")
    assert e <= MATMUL_RTOL


@pytest.mark.parametrize("m", [1, 3, 4, 6])
@pytest.mark.parametrize("rows,cols", [(3000, 4096), (2047, 8192), (600, 28672), (257, 1024), (4100, 128)])
def test_gemv_row_interleave_shapes(rows, cols, m):
    """Row counts that do not divide evenly over the grid's row parts, with
    one, two, four and seven column segments, and x in passes of up to four
    rows."""
    say("gemv shapes", rows, cols, "m", m)
    torch = need_gpu()
    w = syn.normal_f32((rows, cols), 0.02, rows + cols)
    xb = syn.to_bf16(syn.normal_f32((m, cols), 2.0, 63 + m))
    W = nf4.quantize_weight(to_dev(w), double_quant=True)
    y = nf4.nf4_gemv(W, xb.to("cuda"), y_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.matmul_ref(syn.bf16_to_f32(xb), _full_oracle_wdeq(w, True))
    e = oracle.rel_frobenius(_y_f64(y), ref)
    say(f"  rel err {e:.2e}")
    assert e <= MATMUL_RTOL


@pytest.mark.parametrize("m,rows,cols", [(1, 64, 64), (37, 200, 128), (130, 129, 192), (256, 256, 512), (300, 520, 1024)])
@pytest.mark.parametrize("lora", [0, 1, 16])
@pytest.mark.parametrize("dq", [False, True])
def test_gemm_small(m, rows, cols, lora, dq):
    """Fewer tiles than compute units: with more than 128 rows of x each tile
    is cut into two 128-row halves (m = 130: a second half of 2 rows; m = 300:
    the second band's empty half is skipped); m <= 128 keeps whole tiles."""
    say("gemm", m, rows, cols, "lora", lora, "dq" if dq else "plain")
    torch = need_gpu()
    w = syn.normal_f32((rows, cols), 0.02, m + rows + cols)
    xb = syn.to_bf16(syn.normal_f32((m, cols), 1.0, 17 + m))
    W = nf4.quantize_weight(to_dev(w), double_quant=dq)
    a = b = None
    s = 0.0
    if lora:
        a = syn.to_bf16(syn.normal_f32((lora, cols), 0.01, 6))
        b = syn.to_bf16(syn.normal_f32((rows, lora), 0.01, 7))
        s = 32.0 / lora
    y = nf4.nf4_gemm(W, xb.to("cuda"), lora_a=None if a is None else a.to("cuda"),
                     lora_b=None if b is None else b.to("cuda"), lora_scale=s)
    torch.cuda.synchronize()
    _check_gemm(y, xb, _full_oracle_wdeq(w, dq), a, b, s)


@pytest.mark.parametrize("m,rows,cols,r", [(513, 300, 320, 64), (100, 260, 64, 33), (33, 257, 128, 17)])
def test_gemm_lora_ranks(m, rows, cols, r):
    """Largest rank, ranks that are not a multiple of 16, ragged M and N."""
    say("gemm lora rank", r, "shape", m, rows, cols)
    torch = need_gpu()
    w = syn.normal_f32((rows, cols), 0.02, 40 + r)
    xb = syn.to_bf16(syn.normal_f32((m, cols), 1.0, 41 + r))
    a = syn.to_bf16(syn.normal_f32((r, cols), 0.02, 42 + r))
    b = syn.to_bf16(syn.normal_f32((rows, r), 0.02, 43 + r))
    s = 16.0 / r
    W = nf4.quantize_weight(to_dev(w), double_quant=True)
    y = nf4.nf4_gemm(W, xb.to("cuda"), lora_a=a.to("cuda"), lora_b=b.to("cuda"), lora_scale=s)
    torch.cuda.synchronize()
    _check_gemm(y, xb, _full_oracle_wdeq(w, True), a, b, s)


def test_gemm_lora_only_term_and_zero_b():
    """With B = 0 the LoRA path adds nothing; with a one-hot x the product
    returns a dequantized column exactly rounded to bf16 (192 rows of x: both
    halves of a cut tile)."""
    say("gemm closed forms")
    torch = need_gpu()
    rows, cols, m = 192, 256, 192
    w = syn.normal_f32((rows, cols), 0.02, 12)
    W = nf4.quantize_weight(to_dev(w), double_quant=True)
    xb = syn.to_bf16(syn.normal_f32((m, cols), 1.0, 13)).to("cuda")
    a = syn.to_bf16(syn.normal_f32((16, cols), 0.01, 14)).to("cuda")
    zb = torch.zeros((rows, 16), dtype=torch.bfloat16, device="cuda")
    y0 = nf4.nf4_gemm(W, xb)
    y1 = nf4.nf4_gemm(W, xb, lora_a=a, lora_b=zb, lora_scale=2.0)
    e = torch.zeros((m, cols), dtype=torch.bfloat16, device="cuda")
    for i in range(m):
        e[i, (i * 5) % cols] = 1.0
    ye = nf4.nf4_gemm(W, e)
    wdeq = nf4.nf4_dequantize(W, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    for i in range(m):
        assert torch.equal(ye[i], wdeq[:, (i * 5) % cols])
