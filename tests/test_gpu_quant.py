"""GPU parity of nf4_quantize, nf4_double_quant and nf4_dequantize against the
CPU oracle: bit-exact codes, packed bytes, scales, int8 codes, mean and
dequantized values."""

from __future__ import annotations

import numpy as np
import pytest

import dequant_matmul_nf4_amd as nf4
import oracle
import synthetic as syn
from tests.gpu_common import bf16_bits, f32_bits, need_gpu, say, to_dev, u8

pytestmark = pytest.mark.gpu


def _quant_both(x_f32: np.ndarray, as_bf16: bool):
    """Quantize x on the GPU (fp32 or bf16 input) and in the oracle."""
    torch = need_gpu()
    if as_bf16:
        xt = syn.to_bf16(x_f32)
        x_exact = syn.bf16_to_f32(xt)
    else:
        xt = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
        x_exact = x_f32.astype(np.float32)
    packed, absmax = nf4.nf4_quantize(xt.to("cuda"))
    torch.cuda.synchronize()
    p_ref, a_ref = oracle.quantize(x_exact.reshape(-1))
    return packed, absmax, p_ref, a_ref, x_exact


def _assert_quant_equal(packed, absmax, p_ref, a_ref):
    got_p, got_a = u8(packed), f32_bits(absmax)
    if not np.array_equal(got_p, p_ref):
        bad = np.nonzero(got_p != p_ref)[0]
        raise AssertionError(f"{bad.size} packed bytes differ, first at {bad[:5]}: gpu {got_p[bad[:5]]} oracle {p_ref[bad[:5]]}")
    assert np.array_equal(got_a, a_ref.view(np.uint32))


@pytest.mark.parametrize("n", [1, 2, 7, 8, 63, 64, 65, 127, 129, 1000, 4097, 65536 + 33, 1_000_003])
@pytest.mark.parametrize("as_bf16", [False, True])
def test_quantize_ragged_sizes(n, as_bf16):
    say("quantize ragged", n, "bf16" if as_bf16 else "f32")
    x = syn.random_blocks_f32(n, 1000 + n)
    packed, absmax, p_ref, a_ref, _ = _quant_both(x, as_bf16)
    _assert_quant_equal(packed, absmax, p_ref, a_ref)


def test_quantize_c1_fp32_full():
    say("quantize C1 1024x1024 fp32")
    inp = syn.c1_inputs()
    packed, absmax, p_ref, a_ref, _ = _quant_both(inp["w_f32"], False)
    _assert_quant_equal(packed, absmax, p_ref, a_ref)


def test_quantize_c2_bf16_full():
    say("quantize C2 4096x4096 bf16 with outliers")
    torch = need_gpu()
    w = syn.c2_weight()
    packed, absmax = nf4.nf4_quantize(w.to("cuda"))
    torch.cuda.synchronize()
    p_ref, a_ref = oracle.quantize(syn.bf16_to_f32(w).reshape(-1))
    _assert_quant_equal(packed, absmax, p_ref, a_ref)


def _adversarial_blocks() -> np.ndarray:
    cb = oracle.codebook().astype(np.float64)
    blocks = []
    # exact ties at every midpoint that fp32 can hold, at several scales
    for i in range(15):
        m = np.float32((cb[i] + cb[i + 1]) / 2)
        if float(m) != (cb[i] + cb[i + 1]) / 2:
            continue
        for k in (-126, -60, -3, 0, 3, 90):
            s = np.float32(2.0 ** k)
            b = np.zeros(64, np.float32)
            b[0] = s
            b[1] = m * s
            b[2] = -m * s
            b[3] = np.nextafter(m, np.float32(2)) * s
            b[4] = np.nextafter(m, np.float32(-2)) * s
            blocks.append(b)
    # every level exactly, and its neighbours
    for c in cb:
        b = np.zeros(64, np.float32)
        b[0] = 1.0
        b[1] = np.float32(c)
        b[2] = np.nextafter(np.float32(c), np.float32(2))
        b[3] = np.nextafter(np.float32(c), np.float32(-2))
        blocks.append(b)
    blocks.append(np.zeros(64, np.float32))                      # all zero
    z = np.zeros(64, np.float32); z[::2] = -0.0; blocks.append(z)  # negative zeros
    rng = np.random.default_rng(5)
    sub = (rng.standard_normal(64) * 1e-39).astype(np.float32); blocks.append(sub)      # subnormal block
    tiny = np.zeros(64, np.float32); tiny[7] = np.float32(1.4e-45); blocks.append(tiny)  # smallest subnormal
    big = (rng.standard_normal(64) * 1e37).astype(np.float32); blocks.append(big)
    out = (rng.standard_normal(64) * 0.02).astype(np.float32); out[40] = 50.0; blocks.append(out)
    neg = (rng.standard_normal(64) * 0.02).astype(np.float32); neg[3] = -7.0; blocks.append(neg)
    return np.concatenate(blocks)


def test_quantize_adversarial_blocks_fp32():
    say("quantize adversarial fp32")
    x = _adversarial_blocks()
    packed, absmax, p_ref, a_ref, _ = _quant_both(x, False)
    _assert_quant_equal(packed, absmax, p_ref, a_ref)
    # partial last block: drop a few values
    say("quantize adversarial fp32 partial tail")
    packed, absmax, p_ref, a_ref, _ = _quant_both(x[:-13], False)
    _assert_quant_equal(packed, absmax, p_ref, a_ref)


def test_quantize_adversarial_blocks_bf16():
    say("quantize adversarial bf16")
    x = _adversarial_blocks()
    packed, absmax, p_ref, a_ref, _ = _quant_both(x, True)
    _assert_quant_equal(packed, absmax, p_ref, a_ref)


def test_quantize_exhaustive_fp32_decisions():
    """Every fp32 value in [-1, 1] goes through nf4_quantize in blocks whose
    absmax is exactly 1, so the normalized value is the input itself.  The
    nearest-level map is monotone, so the GPU codes must be monotone along the
    sweep and agree with the oracle on both sides of each of their 15 steps."""
    torch = need_gpu()
    per_block = 63
    chunk_blocks = 1 << 21
    for sign in (0, 1):
        say("exhaustive sweep sign", sign)
        lo, hi = 0, 0x3F800000            # bit patterns of +0 .. 1.0 (or -0 .. -1.0)
        total = hi - lo + 1
        prev_last_code = None
        prev_last_val = None
        steps = []
        start = lo
        while start <= hi:
            nb = min(chunk_blocks, -(-(hi - start + 1) // per_block))
            cnt = min(nb * per_block, hi - start + 1)
            bits = torch.arange(start, start + cnt, dtype=torch.int64, device="cuda")
            if sign:
                bits = bits | 0x80000000
            vals = bits.to(torch.int32).view(torch.float32) if not sign else (bits - (1 << 32)).to(torch.int32).view(torch.float32)
            pad = nb * per_block - cnt
            body = torch.cat([vals, torch.zeros(pad, dtype=torch.float32, device="cuda")]).view(nb, per_block)
            ones = torch.ones((nb, 1), dtype=torch.float32, device="cuda")
            x = torch.cat([ones, body], dim=1).contiguous()
            packed, absmax = nf4.nf4_quantize(x)
            assert bool((absmax == 1).all())
            hi_n = (packed >> 4).to(torch.int16)
            lo_n = (packed & 15).to(torch.int16)
            codes = torch.stack([hi_n, lo_n], dim=1).view(nb, 64)[:, 1:].reshape(-1)[:cnt]
            d = codes[1:] - codes[:-1]
            if sign == 0:
                assert bool((d >= 0).all()), "codes not monotone"
            else:
                assert bool((d <= 0).all()), "codes not monotone"
            idx = torch.nonzero(d).reshape(-1)
            for i in idx.tolist():
                steps.append((float(vals[i]), int(codes[i]), float(vals[i + 1]), int(codes[i + 1])))
            if prev_last_code is not None and int(codes[0]) != prev_last_code:
                steps.append((prev_last_val, prev_last_code, float(vals[0]), int(codes[0])))
            prev_last_code, prev_last_val = int(codes[-1]), float(vals[-1])
            start += cnt
            del bits, vals, body, x, packed, absmax, codes, d
        assert total > 1e9
        first = 7
        last = 15 if sign == 0 else 0
        assert len(steps) == abs(last - first), steps
        for a, ca, b, cb_ in steps:
            ref = oracle.nearest_code(np.array([a, b], dtype=np.float32))
            assert (int(ref[0]), int(ref[1])) == (ca, cb_), (a, b, ca, cb_, ref)


@pytest.mark.parametrize("nb", [1, 3, 255, 256, 257, 1000, 16384, 262144 + 77])
def test_double_quant_parity(nb):
    say("double quant nblocks", nb)
    torch = need_gpu()
    rng = np.random.default_rng(nb)
    a = np.abs(rng.standard_normal(nb).astype(np.float32) * np.float32(0.05)) + np.float32(0.01)
    if nb > 300:
        a[rng.integers(0, nb, 20)] *= np.float32(40)
    q, s2, mean = nf4.nf4_double_quant(to_dev(a))
    torch.cuda.synchronize()
    rq, rs2, rmean = oracle.double_quant(a)
    assert f32_bits(mean)[0] == np.float32(rmean).view(np.uint32)
    assert np.array_equal(f32_bits(s2), rs2.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), rq)


def test_double_quant_exact_mean_wide_range():
    """Scales spanning the whole float32 range: the mean must still be the
    correctly rounded mean of the exact sum, whatever the summation order."""
    say("double quant wide range")
    torch = need_gpu()
    rng = np.random.default_rng(77)
    nb = 300_001
    e = rng.integers(-149, 127, nb)
    a = np.ldexp(rng.uniform(1, 2, nb), e).astype(np.float32)
    a[::1000] = 0.0
    a[5] = np.float32(3.4e38)
    a[6] = np.float32(1.4e-45)
    q, s2, mean = nf4.nf4_double_quant(to_dev(a))
    torch.cuda.synchronize()
    rq, rs2, rmean = oracle.double_quant(a)
    assert f32_bits(mean)[0] == np.float32(rmean).view(np.uint32)
    assert np.array_equal(f32_bits(s2), rs2.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), rq)


def test_double_quant_c2_pipeline():
    say("quantize + double quant C2")
    torch = need_gpu()
    w = syn.c2_weight()
    packed, absmax = nf4.nf4_quantize(w.to("cuda"))
    q, s2, mean = nf4.nf4_double_quant(absmax)
    torch.cuda.synchronize()
    ra = oracle.block_absmax(syn.bf16_to_f32(w).reshape(-1))
    rq, rs2, rmean = oracle.double_quant(ra)
    assert f32_bits(mean)[0] == np.float32(rmean).view(np.uint32)
    assert np.array_equal(f32_bits(s2), rs2.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), rq)


@pytest.mark.parametrize("shape", [(1, 1), (1, 63), (3, 65), (17, 128), (1024, 1024), (257, 4096)])
@pytest.mark.parametrize("dq", [False, True])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_parity(shape, dq, out):
    say("dequantize", shape, "dq" if dq else "plain", out)
    torch = need_gpu()
    rows, cols = shape
    x = syn.normal_f32(shape, 0.02, rows * 31 + cols)
    if x.size > 100:
        x.reshape(-1)[:: 997] *= np.float32(20)
    xt = to_dev(x)
    w = nf4.quantize_weight(xt, double_quant=dq)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y = nf4.nf4_dequantize(w, out_dtype=dt)
    torch.cuda.synchronize()
    p_ref, a_ref = oracle.quantize(x.reshape(-1))
    if dq:
        rq, rs2, rmean = oracle.double_quant(a_ref)
        ref = oracle.dequantize(p_ref, x.size, qabsmax=rq, absmax2=rs2, mean=rmean, out=out)
    else:
        ref = oracle.dequantize(p_ref, x.size, absmax=a_ref, out=out)
    got = bf16_bits(y).reshape(-1) if out == "bf16" else f32_bits(y).reshape(-1)
    want = ref if out == "bf16" else ref.view(np.uint32)
    assert np.array_equal(got, want)


def test_quantize_deterministic():
    say("quantize determinism")
    torch = need_gpu()
    w = syn.c2_weight(1024, 4096).to("cuda")
    p1, a1 = nf4.nf4_quantize(w)
    q1, s1, m1 = nf4.nf4_double_quant(a1)
    p2, a2 = nf4.nf4_quantize(w)
    q2, s2, m2 = nf4.nf4_double_quant(a2)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(a1, a2)
    assert torch.equal(q1, q2) and torch.equal(s1, s2) and torch.equal(m1, m2)


@pytest.mark.parametrize("kind", ["wide", "narrow_with_outliers", "with_zeros"])
def test_double_quant_large_scale_arrays_bit_exact(kind):
    """Scale arrays large enough (>= 8 per summing thread) for the partial-sum
    kernel's three-digit window: scales spread over many exponent ranges
    (most contributions fall outside any one window), scales in one range
    with rare outliers, and runs of zero scales -- mean, codes and group
    scales bit-exact against the oracle."""
    say("double quant large", kind)
    torch = need_gpu()
    nb = 600_000
    rng = np.random.default_rng({"wide": 41, "narrow_with_outliers": 42, "with_zeros": 43}[kind])
    if kind == "wide":
        a = np.exp2(rng.uniform(-100, 60, nb)) * rng.uniform(1, 2, nb)
    elif kind == "narrow_with_outliers":
        a = rng.uniform(0.04, 0.09, nb)
        idx = rng.choice(nb, 50, replace=False)
        a[idx] = np.exp2(rng.uniform(-120, 100, idx.size))
    else:
        a = rng.uniform(0.01, 0.5, nb)
        a[rng.random(nb) < 0.3] = 0.0
        a[:70_000] = 0.0
    a = a.astype(np.float32)
    q, s2, mean = nf4.nf4_double_quant(torch.from_numpy(a).to("cuda"))
    torch.cuda.synchronize()
    q_o, s2_o, mean_o = oracle.double_quant(a)
    assert f32_bits(mean)[0] == np.float32(mean_o).view(np.uint32)
    assert np.array_equal(q.cpu().numpy(), q_o)
    assert np.array_equal(f32_bits(s2), s2_o.view(np.uint32))


def _threshold_inputs(levels_ascending: np.ndarray, seed: int) -> np.ndarray:
    """Blocks whose absmax a has a random odd significand (so 1/a is not
    exact and the kernel's reciprocal-based division has a residual to
    correct) and whose other 63 values sit where fl32(x / a) lands within a
    few ulps of a decision threshold (the midpoint of two neighbouring
    levels): x = fl32(a * t) for t at -4 .. +4 ulps of each midpoint, and the
    float32 neighbours of each such x.  The exponents of a span the range the
    kernel divides by reciprocal (2^-98 <= a < 2^126) and both sides beyond
    it, where it divides per value, including subnormal a.  Half of the blocks
    hold -a as their largest magnitude."""
    rng = np.random.default_rng(seed)
    lv = levels_ascending.astype(np.float64)
    mids = (lv[:-1] + lv[1:]) / 2
    t = []
    for m in mids:
        c = np.float32(m)
        for k in range(-4, 5):
            v = c
            for _ in range(abs(k)):
                v = np.nextafter(v, np.float32(np.inf) if k > 0 else np.float32(-np.inf))
            t.append(v)
    t = np.array(t, dtype=np.float32)
    exps = [-126, -120, -99, -98, -97, -60, -10, -1, 0, 1, 10, 60, 100, 124, 125, 126, 127]
    avals = []
    for e in exps:
        for _ in range(6):
            sig = 1.0 + (2 * int(rng.integers(0, 1 << 22)) + 1) * 2.0 ** -23
            avals.append(np.float32(np.ldexp(sig, e)))
    for e in (-130, -140, -148):  # subnormal a
        avals.append(np.float32(np.ldexp(1.0 + (2 * int(rng.integers(0, 1 << 20)) + 1) * 2.0 ** -21, e)))
    blocks = []
    for i, a in enumerate(avals):
        x = (np.float32(a) * t).astype(np.float32)
        vals = np.concatenate([x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(-np.inf))])
        vals = vals[np.abs(vals) <= a]
        for j in range(0, vals.size, 63):
            body = np.zeros(63, dtype=np.float32)
            part = vals[j:j + 63]
            body[:part.size] = part
            head = np.float32(-a) if (i + j // 63) % 2 else np.float32(a)
            blocks.append(np.concatenate([[head], body]).astype(np.float32))
    return np.concatenate(blocks)


@pytest.mark.parametrize("kind", ["nf4", "fp4"])
def test_quantize_division_near_every_threshold(kind):
    """Bit-exact codes where the normalized value is within a few ulps of a
    decision threshold, for scales that are not powers of two: a wrong last
    bit in fl32(x / a) flips the code there."""
    torch = need_gpu()
    if kind == "nf4":
        levels = oracle.codebook()
    else:
        lv = oracle.fp4_codebook()
        levels = np.unique(lv[oracle.FP4_PRODUCED])
    x = _threshold_inputs(levels, 11 if kind == "nf4" else 12)
    say("quantize near thresholds", kind, "values", x.size)
    xt = torch.from_numpy(x).to("cuda")
    packed, absmax = nf4.nf4_quantize(xt, fp4=kind == "fp4")
    torch.cuda.synchronize()
    p_ref, a_ref = oracle.quantize(x, kind=kind)
    _assert_quant_equal(packed, absmax, p_ref, a_ref)
    # the sweep does reach both division paths and every threshold
    a = np.abs(x.reshape(-1, 64)[:, 0])
    assert ((a >= 2.0 ** -98) & (a < 2.0 ** 126)).any() and ((a < 2.0 ** -98) | (a >= 2.0 ** 126)).any()
