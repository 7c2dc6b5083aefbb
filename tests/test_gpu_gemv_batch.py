"""GPU parity of nf4_gemv_batched, the decode GEMV of several weights in one
launch (bitsandbytes tool page, "How it works", Step 5).

Every output is compared with the oracle's float64 product of its float32
dequantized weight (gpu_common.check_full_product: whole-output and
per-64-output relative Frobenius error <= 1e-2 plus the per-element bound;
the decode kernels take the levels rounded to fp16, a 2^-11 relative weight
term).  Each output is also bit-identical to nf4_gemv on the same weight and
x: the batched launch changes the schedule, not the arithmetic."""

from __future__ import annotations

import numpy as np
import pytest

import dequant_matmul_nf4_amd as nf4
import oracle
import synthetic as syn
from tests.gpu_common import check_full_product, need_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _oracle_f32(w: np.ndarray, dq: str, qt: str = "nf4") -> np.ndarray:
    p, a = oracle.quantize(w.reshape(-1), kind=qt)
    if dq == "plain":
        return oracle.dequantize(p, w.size, absmax=a, out="f32", kind=qt).reshape(w.shape)
    if dq == "fp8":
        q, s2, mean = oracle.double_quant_f8(a)
        return oracle.dequantize(p, w.size, qabsmax=q, absmax2=s2, mean=mean, out="f32", dq_kind="fp8",
                                 kind=qt).reshape(w.shape)
    q, s2, mean = oracle.double_quant(a)
    return oracle.dequantize(p, w.size, qabsmax=q, absmax2=s2, mean=mean, out="f32", kind=qt).reshape(w.shape)


def _run(shapes, x_of, dq="int8", y_dtype="bf16", seed=0, qt="nf4"):
    """Quantizes one weight per shape (code book qt), multiplies them in one
    batched call (weight i takes x number x_of[i]) and checks every output."""
    torch = need_gpu()
    ws_np = [syn.normal_f32(sh, 0.02, 900 + seed + 17 * i) for i, sh in enumerate(shapes)]
    Ws = [nf4.quantize_weight(to_dev(w), double_quant=dq != "plain", dq_type="fp8" if dq == "fp8" else "int8",
                              quant_type=qt)
          for w in ws_np]
    cols_of_x = {}
    for i, sh in enumerate(shapes):
        cols_of_x.setdefault(x_of[i], sh[1])
        assert cols_of_x[x_of[i]] == sh[1]
    xs_b = {k: syn.to_bf16(syn.normal_f32((1, c), 1.0, 950 + seed + k)) for k, c in cols_of_x.items()}
    xs_d = {k: v.to("cuda") for k, v in xs_b.items()}
    ydt = torch.bfloat16 if y_dtype == "bf16" else torch.float32
    ys = nf4.nf4_gemv_batched(Ws, [xs_d[k] for k in x_of], y_dtype=ydt)
    single = [nf4.nf4_gemv(W, xs_d[k], y_dtype=ydt) for W, k in zip(Ws, x_of)]
    again = nf4.nf4_gemv_batched(Ws, [xs_d[k] for k in x_of], y_dtype=ydt)
    torch.cuda.synchronize()
    for i, (y, y1, y2) in enumerate(zip(ys, single, again)):
        assert torch.equal(y, y1), f"weight {i}: batched and single launches differ"
        assert torch.equal(y, y2), f"weight {i}: not deterministic"
    for i, (w, y) in enumerate(zip(ws_np, ys)):
        wdeq = _oracle_f32(w, dq, qt)
        xf = syn.bf16_to_f32(xs_b[x_of[i]])
        ref = oracle.matmul_ref(xf, wdeq)
        sabs = np.abs(xf).astype(np.float64) @ np.abs(wdeq).astype(np.float64).T
        got = y.to(torch.float32).cpu().numpy().astype(np.float64)
        check_full_product(got, ref, sabs, terms=w.shape[1], tile=(1, 64), w_rel=2.0 ** -11, label=f"weight {i}")


def test_batched_shared_and_distinct_x_mixed_widths():
    """Seven weights: three sharing one x (one, two and seven column
    segments of different heights), two sharing another, two on their own;
    ragged row counts."""
    say("gemv batched: mixed widths and shared x")
    _run([(300, 4096), (77, 4096), (1024, 4096), (2000, 8192), (129, 8192), (520, 28672), (64, 64)],
         [0, 0, 0, 1, 1, 2, 3])


@pytest.mark.parametrize("dq", ["plain", "int8", "fp8"])
@pytest.mark.parametrize("y_dtype", ["bf16", "f32"])
def test_batched_scale_forms_and_outputs(dq, y_dtype):
    say("gemv batched:", dq, y_dtype)
    _run([(1000, 1024), (257, 2048), (33, 1024)], [0, 1, 0], dq=dq, y_dtype=y_dtype, seed=5)


@pytest.mark.parametrize("dq", ["plain", "int8"])
def test_batched_fp4_code_book(dq):
    """Weights quantized with the FP4 code book (bitsandbytes tool page,
    "What it is", read as the E2M1 levels): the batched launch takes the code
    book from the weights, which must all share it."""
    say("gemv batched: fp4", dq)
    _run([(700, 2048), (129, 1024), (64, 2048)], [0, 1, 0], dq=dq, seed=21, qt="fp4")


def test_batched_single_weight_and_eight_weights():
    say("gemv batched: 1 and 8 weights")
    _run([(4099, 4096)], [0], seed=11)
    _run([(256 + 37 * i, 1024 * (1 + i % 3)) for i in range(8)], [i % 3 for i in range(8)], seed=12)


def test_batched_wide_and_many_distinct_x():
    """Four distinct x of 16384 values each, and a weight 49152 wide between
    two narrow ones (each wave takes its x slice of every group from global
    memory as it enters the group)."""
    say("gemv batched: wide and many distinct x")
    _run([(300, 16384), (200, 16384), (100, 16384), (50, 16384)], [0, 1, 2, 3], seed=13)
    _run([(64, 1024), (100, 49152), (70, 2048)], [0, 1, 2], seed=14)


def test_batched_70b_layer_bit_identical_to_single_launches():
    """The seven matrices of a 70B-shaped layer (drawn on the device exactly
    as the benchmark draws them) in one call, with q, k, v, o, gate, up
    sharing one x:
    every output bit-identical to nf4_gemv on the same weight; the q
    projection also against the oracle on every output."""
    torch = need_gpu()
    say("gemv batched: 70B-shaped layer")
    g = torch.Generator(device="cuda")
    g.manual_seed(5_000_009)
    x8 = torch.randn((1, 8192), generator=g, device="cuda").to(torch.bfloat16)
    x28 = torch.randn((1, 28672), generator=g, device="cuda").to(torch.bfloat16)
    Ws, xs = [], []
    for name in syn.C5_ORDER:
        w = syn.c5_weight_device(0, name)
        Ws.append(nf4.quantize_weight(w, double_quant=True))
        xs.append(x28 if w.shape[1] == 28672 else x8)
        if name == "q":
            wq = syn.bf16_to_f32(w)
        del w
    ys = nf4.nf4_gemv_batched(Ws, xs)
    ys_f = nf4.nf4_gemv_batched(Ws, xs, y_dtype=torch.float32)
    single = [nf4.nf4_gemv(W, x) for W, x in zip(Ws, xs)]
    torch.cuda.synchronize()
    for name, y, y1 in zip(syn.C5_ORDER, ys, single):
        assert torch.equal(y, y1), name
    wdeq = _oracle_f32(wq, "int8")
    xf = syn.bf16_to_f32(x8)
    ref = oracle.matmul_ref(xf, wdeq)
    sabs = np.abs(xf).astype(np.float64) @ np.abs(wdeq).astype(np.float64).T
    check_full_product(ys_f[0].cpu().numpy().astype(np.float64), ref, sabs, terms=8192, tile=(1, 64),
                       w_rel=2.0 ** -11, label="q (f32 out)")
