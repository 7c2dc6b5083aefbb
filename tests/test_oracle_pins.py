"""Pins for the CPU oracle: checks against closed forms, exact rational
arithmetic, brute force on tiny inputs, library routines and the worked
example printed on the pages.  None of these calls the HIP library."""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synthetic import normal_f32, random_blocks_f32
from tests.exact import frac, nearest_level_exact, rn32, rn64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- P1 code book

def test_codebook_invariants():
    cb = oracle.codebook()
    assert cb.dtype == np.float32 and cb.shape == (16,)
    assert np.all(np.diff(cb.astype(np.float64)) > 0)
    assert cb[0] == np.float32(-1.0) and cb[15] == np.float32(1.0)
    assert cb[7] == np.float32(0.0) and not np.signbit(cb[7])
    assert (cb < 0).sum() == 7 and (cb > 0).sum() == 8


def test_codebook_two_inverse_normal_routines_agree():
    a = oracle.levels_f64(oracle.inv_phi_bisect)
    b = oracle.levels_f64(oracle.inv_phi_stdlib)
    assert np.max(np.abs(a - b)) <= 1e-15
    assert np.array_equal(a.astype(np.float32), b.astype(np.float32))
    # each float64 level sits far from an fp32 rounding boundary compared with
    # the ~1e-15 disagreement, so the fp32 rounding is determined
    for v in a:
        if v in (0.0, 1.0, -1.0):
            continue
        f = np.float32(v)
        up = float(np.nextafter(f, np.float32(2)))
        dn = float(np.nextafter(f, np.float32(-2)))
        margin = min(abs(v - (float(f) + up) / 2), abs(v - (float(f) + dn) / 2))
        assert margin / abs(v) > 1e-12


def test_codebook_equal_share_of_bell_curve():
    """Forward check: Phi(level * Phi^{-1}(delta)) lands on evenly spaced
    probabilities on each side ("each covers an equal share of that bell curve")."""
    top = oracle.inv_phi_bisect(oracle.DELTA)
    cb = oracle.codebook().astype(np.float64)
    phi = lambda z: 0.5 * math.erfc(-z / math.sqrt(2.0))
    delta = float(oracle.DELTA)
    pos = sorted([phi(c * top) for c in cb[8:]], reverse=True)     # 8 values
    neg = sorted([phi(-c * top) for c in cb[:7]], reverse=True)    # 7 values
    step_pos = (delta - 0.5) / 8
    step_neg = (delta - 0.5) / 7
    for i, p in enumerate(pos):
        assert abs(p - (delta - i * step_pos)) < 2e-7
    for j, p in enumerate(neg):
        assert abs(p - (delta - j * step_neg)) < 2e-7
    assert abs(phi(0.0) - 0.5) == 0.0


# ----------------------------------------------------- P2 division and nearest

def test_fp32_division_is_correctly_rounded():
    # the quantizer's domain: |x| <= a, including subnormal quotients
    x = random_blocks_f32(3000, 12)
    y = random_blocks_f32(3000, 13)
    a = np.maximum(np.abs(x), np.abs(y)).astype(np.float32)
    a[a == 0] = np.float32(1.0)
    with np.errstate(under="ignore"):
        q = (x / a).astype(np.float32)
    for xi, ai, qi in zip(x, a, q):
        assert rn32(frac(xi) / frac(ai)) == qi


def _brute_quantize(block):
    lv = oracle.codebook()
    a = max(abs(frac(v)) for v in block)
    codes = []
    for v in block:
        if a == 0:
            codes.append(7)
            continue
        n = rn32(frac(v) / a)
        codes.append(nearest_level_exact(frac(n), lv))
    return codes, np.float32(float(a))


@pytest.mark.parametrize("seed", range(6))
def test_quantize_matches_brute_force_on_tiny_blocks(seed):
    rng = np.random.default_rng(100 + seed)
    size = int(rng.integers(2, 65))
    kind = ["normal", "uniform", "wide"][seed % 3]
    x = random_blocks_f32(size, 200 + seed, kinds=(kind,))
    packed, absmax = oracle.quantize(x)
    codes = oracle.unpack(packed, x.size)
    bcodes, ba = _brute_quantize(list(x))
    assert absmax.shape == (1,) and absmax[0] == ba
    assert list(codes) == bcodes


def _representable_midpoints():
    cb = oracle.codebook()
    out = []
    for i in range(15):
        m = (frac(cb[i]) + frac(cb[i + 1])) / 2
        if Fraction(float(rn32(m))) == m:      # exactly representable in fp32
            out.append((i, m))
    return out


def test_ties_go_away_from_zero():
    mids = _representable_midpoints()
    assert len(mids) >= 1
    for i, m in mids:
        for k in (-3, 0, 5):
            scale = Fraction(2) ** k
            block = np.array([float(m * scale), float(scale), -float(scale) / 2], dtype=np.float32)
            packed, absmax = oracle.quantize(block)
            code = oracle.unpack(packed, 3)[0]
            expect = i + 1 if m > 0 else i   # the level farther from zero
            assert code == expect, (i, float(m), k)
            assert nearest_level_exact(m, oracle.codebook()) == expect


def test_nearest_code_vs_exact_on_neighbourhoods_of_midpoints():
    cb = oracle.codebook()
    vals = []
    for i in range(15):
        m = np.float32((float(cb[i]) + float(cb[i + 1])) / 2)
        v = m
        for _ in range(3):
            v = np.nextafter(v, np.float32(-2))
        for _ in range(7):
            vals.append(v)
            v = np.nextafter(v, np.float32(2))
    vals = np.array(vals, dtype=np.float32)
    got = oracle.nearest_code(vals)
    for v, g in zip(vals, got):
        assert g == nearest_level_exact(frac(v), cb)


# ------------------------------------------------------------ P3 round trips

def test_round_trip_levels_at_powers_of_two():
    cb = oracle.codebook()
    for i, c in enumerate(cb):
        for k in (-20, -3, 0, 7):
            a = np.float32(2.0 ** k)
            top = a if c >= 0 else -a
            block = np.array([np.float32(c) * a, top] + [0] * 62, dtype=np.float32)
            packed, absmax = oracle.quantize(block)
            codes = oracle.unpack(packed, 64)
            assert codes[0] == i
            w = oracle.dequantize(packed, 64, absmax=absmax)
            assert w[0] == np.float32(c) * a
            assert w[1] == top


def test_block_max_maps_to_plus_minus_absmax_and_zero_block():
    x = normal_f32((64 * 50,), 0.02, 77)
    packed, absmax = oracle.quantize(x)
    codes = oracle.unpack(packed, x.size).reshape(50, 64)
    w = oracle.dequantize(packed, x.size, absmax=absmax).reshape(50, 64)
    xb = x.reshape(50, 64)
    for b in range(50):
        j = int(np.argmax(np.abs(xb[b])))
        assert codes[b, j] in (0, 15)
        assert abs(w[b, j]) == absmax[b]
        norm = oracle.normalize(xb[b], absmax[b:b + 1])
        assert np.all(np.abs(norm) <= 1)
    z = np.zeros(64, dtype=np.float32)
    z[3] = -0.0
    packed, absmax = oracle.quantize(z)
    assert absmax[0] == 0 and np.all(oracle.unpack(packed, 64) == 7)
    assert np.all(oracle.dequantize(packed, 64, absmax=absmax) == 0)


# ------------------------------------------------------------- P4 packing

def test_pack_closed_form_and_odd_tail():
    codes = np.array([1, 2, 3, 4, 5], dtype=np.uint8)
    assert list(oracle.pack(codes)) == [0x12, 0x34, 0x57]
    x = normal_f32((131,), 1.0, 5)
    packed, absmax = oracle.quantize(x)
    assert packed.size == 66 and absmax.size == 3
    assert packed[-1] & 0xF == 7
    # the partial last block's absmax covers only its valid elements
    assert absmax[2] == np.max(np.abs(x[128:]))


def test_storage_sizes():
    for n in (1, 63, 64, 65, 16384, 16385, 1 << 24):
        nb = -(-n // 64)
        s = oracle.storage_bytes(n, False)
        assert s == {"packed": -(-n // 2), "absmax": 4 * nb}
        s = oracle.storage_bytes(n, True)
        assert s == {"packed": -(-n // 2), "qabsmax": nb, "absmax2": 4 * (-(-nb // 256)), "mean": 4}


# ------------------------------------------------------ P5 footprint closed form

def test_footprint_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "footprint.json")))
    n = 1 << 24
    assert oracle.bits_per_param(n, False) == 4.5
    assert abs(oracle.bits_per_param(n, True) - (4 + 8 / 64 + 32 / 16384 + 32 / n)) < 1e-12
    p = g["params"]
    fp16 = 2 * p / 1e9
    nf4 = sum(oracle.storage_bytes(p, False).values()) / 1e9
    nf4_dq = sum(oracle.storage_bytes(p, True).values()) / 1e9
    codes_only = oracle.storage_bytes(p, False)["packed"] / 1e9
    assert fp16 == g["fp16_GB"]
    assert codes_only == g["nf4_codes_only_GB"]
    assert abs(nf4 - g["nf4_GB_approx"]) < 0.1          # 3.94 GB ~ "~4 GB"
    assert nf4_dq < nf4 and abs(nf4_dq - 3.61) < 0.01
    saving = oracle.bits_per_param(p, False) - oracle.bits_per_param(p, True)
    assert abs(saving - 0.373) < 0.001 and abs(saving - g["dq_saving_bits_approx"]) < 0.05


# ------------------------------------------------------ P6 int8 worked example

def test_int8_step_reproduces_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "int8_worked_example.json")))
    block = np.array(g["block"], dtype=np.float32)
    q, s = oracle.int8_absmax_quantize(block, blocksize=4)
    assert s[0] == np.float32(g["absmax"])
    norm = (block / s[0]).astype(np.float32)
    assert list(norm) == [np.float32(v) for v in g["normalized"]]
    t = norm * np.float32(127)
    assert np.allclose(t, g["times_127_printed"], atol=0.005)
    assert list(q) == g["q"]
    deq = oracle.dequant_scales(q, s, np.float32(0.0), blocksize2=4)
    for key, printed in g["dequant_printed"].items():
        i = g["q"].index(int(key))
        assert round(float(deq[i]), 4) == printed
        err = abs(float(deq[i]) - g["block"][i])
        assert abs(err - g["abs_error_printed"][key]) < 0.0006


def _half_case(k):
    """An fp32 r with fl32(r * 127) == k + 1/2 exactly."""
    target = np.float32(k + 0.5)
    r = np.float32((k + 0.5) / 127)
    for _ in range(64):
        t = np.float32(r * np.float32(127))
        if t == target:
            return r
        r = np.nextafter(r, np.float32(2) if t < target else np.float32(-2))
    return None


def test_int8_rounds_half_away_from_zero_not_to_even():
    found = 0
    for k in range(2, 126, 2):
        r = _half_case(k)
        if r is None:
            continue
        found += 1
        q, _ = oracle.int8_absmax_quantize(np.array([r, -r, 1.0], dtype=np.float32), 3)
        assert q[0] == k + 1 and q[1] == -(k + 1), k    # half-even would give k
    assert found >= 3


# ---------------------------------------------------------------- P7 DQ

def test_mean_is_the_correctly_rounded_exact_mean():
    for seed in range(3):
        a = np.abs(normal_f32((5000 + seed,), 0.05, 300 + seed)) + np.float32(0.001)
        if seed == 2:
            a[:10] = np.float32(1e-30)     # wide dynamic range: naive sums lose bits
            a[10] = np.float32(3e4)
        exact = sum((Fraction(float(v)) for v in a), Fraction(0))
        want = rn32(Fraction(rn64(Fraction(rn64(exact)) / a.size)))
        assert oracle.exact_mean_f32(a) == want


def test_double_quant_invariants_and_exact_scale_arithmetic():
    x = normal_f32((256 * 64 * 5 + 64 * 3,), 0.02, 41)
    _, absmax = oracle.quantize(x)
    q, s2, mean = oracle.double_quant(absmax)
    nb = absmax.size
    assert q.dtype == np.int8 and q.size == nb and s2.size == -(-nb // 256)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    groups = [q[g * 256:(g + 1) * 256] for g in range(s2.size)]
    for g, s in zip(groups, s2):
        if s > 0:
            assert np.max(np.abs(g.astype(np.int32))) == 127
    a_hat = oracle.dequant_scales(q, s2, mean)
    gidx = np.arange(nb) // 256
    bound = s2[gidx].astype(np.float64) / 254 + 4 * np.spacing(np.abs(absmax).astype(np.float32)).astype(np.float64) + 1e-7
    assert np.all(np.abs(a_hat.astype(np.float64) - absmax) <= bound)
    # each of the three float32 operations, recomputed with exact rationals
    for i in range(0, nb, 97):
        t = rn32(Fraction(int(q[i]), 127))
        t = rn32(frac(t) * frac(s2[gidx[i]]))
        t = rn32(frac(t) + frac(mean))
        assert a_hat[i] == t
    # int8 codes recomputed with exact rationals
    c = (absmax - mean).astype(np.float32)
    for i in range(0, nb, 89):
        s = s2[gidx[i]]
        t = rn32(frac(rn32(frac(c[i]) / frac(s))) * 127) if s > 0 else 0
        r = frac(t)
        want = 0 if s == 0 else int(math.copysign(math.floor(abs(r) + Fraction(1, 2)), float(r)))
        assert q[i] == want


# ---------------------------------------------------------- P8 block locality

def test_block_locality_without_double_quant():
    x = normal_f32((64 * 40,), 0.02, 55)
    p0, a0 = oracle.quantize(x)
    y = x.copy()
    y[64 * 17 + 5] = np.float32(3.0)
    p1, a1 = oracle.quantize(y)
    c0 = oracle.unpack(p0, x.size).reshape(40, 64)
    c1 = oracle.unpack(p1, x.size).reshape(40, 64)
    changed = np.where(np.any(c0 != c1, axis=1) | (a0 != a1))[0]
    assert list(changed) == [17]


# ------------------------------------------------------------- bf16 rounding

def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    v = np.concatenate([random_blocks_f32(20000, 9),
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.4e38, 1e-40, -0.0, 0.0], dtype=np.float32)])
    ours = oracle.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = oracle.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(v).to(torch.bfloat16).float().numpy())


# -------------------------------------------------------------- P9 matmul

def test_matmul_ref_brute_force_and_closed_forms():
    rng = np.random.default_rng(3)
    m, n, k, r = 3, 5, 7, 2
    x = rng.standard_normal((m, k))
    w = rng.standard_normal((n, k))
    a = rng.standard_normal((r, k))
    b = rng.standard_normal((n, r))
    s = 2.0
    y = oracle.matmul_ref(x, w, a, b, s)
    for i in range(m):
        for j in range(n):
            base = sum(x[i, t] * w[j, t] for t in range(k))
            lora = sum(sum(x[i, t] * a[q, t] for t in range(k)) * b[j, q] for q in range(r))
            assert abs(y[i, j] - (base + s * lora)) < 1e-12
    # one-hot rows return columns of W; ones return row sums; B = 0 drops LoRA
    e = np.eye(k)
    assert np.array_equal(oracle.matmul_ref(e, w), w.T)
    assert np.allclose(oracle.matmul_ref(np.ones((1, k)), w)[0], w.sum(axis=1), rtol=0, atol=1e-12)
    assert np.array_equal(oracle.matmul_ref(x, w, a, np.zeros_like(b), s), oracle.matmul_ref(x, w))
    # rank-1 LoRA is an outer product
    a1, b1 = a[:1], b[:, :1]
    d = oracle.matmul_ref(x, w, a1, b1, s) - oracle.matmul_ref(x, w)
    assert np.allclose(d, s * np.outer(x @ a1[0], b1[:, 0]), atol=1e-12)


def test_dequantize_matches_per_element_exact_product():
    x = normal_f32((64 * 9 + 13,), 0.02, 61)
    packed, absmax = oracle.quantize(x)
    w = oracle.dequantize(packed, x.size, absmax=absmax)
    wb = oracle.dequantize(packed, x.size, absmax=absmax, out="bf16")
    cb = oracle.codebook()
    codes = oracle.unpack(packed, x.size)
    for i in range(0, x.size, 7):
        want = rn32(frac(cb[codes[i]]) * frac(absmax[i // 64]))
        assert w[i] == want
        # bf16 = nearest-even 8-bit-significand value of the float32 product
        bf = oracle.bf16_bits_to_f32(wb[i:i + 1])[0]
        assert abs(frac(bf) - frac(want)) <= abs(frac(want)) * Fraction(1, 256)


def test_rel_frobenius():
    assert oracle.rel_frobenius([3.0, 4.0], [3.0, 4.0]) == 0.0
    assert abs(oracle.rel_frobenius([3.0, 4.5], [3.0, 4.0]) - 0.1) < 1e-15


# ------------------------------------------------------------- NEXT-2 LoRA merge

def _round_exact(x: Fraction, man_bits: int, emin: int) -> Fraction:
    """Round-to-nearest-even of a rational into a binary format with
    man_bits significant bits and smallest normal exponent emin (subnormals
    below it), by integer arithmetic on the exact value."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    ax = abs(x)
    e = ax.numerator.bit_length() - ax.denominator.bit_length()
    if Fraction(2) ** e > ax:
        e -= 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - man_bits + 1)
    q = ax / quantum
    lo = q.numerator // q.denominator
    rem = q - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * quantum


def _bf16_bits_of(v: Fraction, negative: bool = False) -> int:
    if v == 0:
        return 0x8000 if negative else 0
    f = np.float32(float(v))  # exact: v is on the bf16 grid
    assert Fraction(float(f)) == v
    return int(f.view(np.uint32)) >> 16


def _f16_bits_of(v: Fraction, negative: bool = False) -> int:
    if v == 0:
        return 0x8000 if negative else 0
    h = np.float16(float(v))
    assert Fraction(float(h)) == v
    return int(h.view(np.uint16))


def _f64_cases():
    rng = np.random.default_rng(5)
    mags = np.exp2(rng.uniform(-30, 12, 4000))
    v = (mags * rng.choice([-1.0, 1.0], 4000)).astype(np.float64)
    # exact ties and their float64 neighbours, for bf16 (8 bits) and fp16 (11 bits)
    extra = []
    for bits in (8, 11):
        base = rng.integers(1 << (bits - 1), 1 << bits, 200).astype(np.float64)
        for t in (base + 0.5) * np.exp2(rng.integers(-20, 4, 200) - bits):
            extra += [t, np.nextafter(t, 0.0), np.nextafter(t, np.inf), -t]
    # fp16 subnormal range
    extra += list(rng.uniform(-6.2e-5, 6.2e-5, 500)) + [2.0 ** -24 * 0.5, 2.0 ** -24 * 1.5, 2.0 ** -25 + 2.0 ** -60]
    return np.concatenate([v, np.array(extra, dtype=np.float64)])


def test_f64_to_bf16_and_f16_round_once_to_nearest_even():
    """Both conversions equal the correctly rounded exact value (rational
    arithmetic), ties to even included, fp16 subnormals included."""
    v = _f64_cases()
    bf = oracle.f64_to_bf16_bits(v)
    hf = oracle.f64_to_f16_bits(v)
    for i, x in enumerate(v):
        fx = Fraction(float(x))
        assert int(bf[i]) == _bf16_bits_of(_round_exact(fx, 8, -126), x < 0), x
        assert int(hf[i]) == _f16_bits_of(_round_exact(fx, 11, -14), x < 0), x


def test_lora_merge_closed_forms():
    """B = 0 gives the dequantized base rounded once (the bf16 dequantize
    output); rank 1 with power-of-two adapters gives deq + s*b*a exactly."""
    rng = np.random.default_rng(11)
    deq = (rng.standard_normal((6, 64)) * 0.02).astype(np.float32)
    a = (rng.standard_normal((3, 64)) * 0.01).astype(np.float32)
    a = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(a))
    zero_b = np.zeros((6, 3), dtype=np.float32)
    assert np.array_equal(oracle.lora_merge(deq, a, zero_b, 2.0, "bf16"), oracle.f32_to_bf16_bits(deq))
    assert np.array_equal(oracle.lora_merge(deq, a, zero_b, 2.0, "f16"), deq.astype(np.float16).view(np.uint16))
    a1 = np.full((1, 64), 2.0 ** -7, dtype=np.float32)
    b1 = np.full((6, 1), 2.0 ** -5, dtype=np.float32)
    expect = deq.astype(np.float64) + 2.0 * 2.0 ** -12
    assert np.array_equal(oracle.lora_merge(deq, a1, b1, 2.0, "bf16"), oracle.f64_to_bf16_bits(expect))


def test_lora_merge_is_the_rounded_exact_value():
    """For bf16 adapters the float64 evaluation is exact, so the merge equals
    the exact rational value rounded once -- checked element by element."""
    rng = np.random.default_rng(12)
    rows, cols, r = 5, 64, 16
    deq = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    a = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits((rng.standard_normal((r, cols)) * 0.01).astype(np.float32)))
    b = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits((rng.standard_normal((rows, r)) * 0.01).astype(np.float32)))
    s = 2.0
    got_b = oracle.lora_merge(deq, a, b, s, "bf16")
    got_h = oracle.lora_merge(deq, a, b, s, "f16")
    for n in range(rows):
        for k in range(cols):
            x = Fraction(float(deq[n, k])) + Fraction(s) * sum(
                Fraction(float(b[n, j])) * Fraction(float(a[j, k])) for j in range(r))
            assert int(got_b[n, k]) == _bf16_bits_of(_round_exact(x, 8, -126), x < 0)
            assert int(got_h[n, k]) == _f16_bits_of(_round_exact(x, 11, -14), x < 0)


# ------------------------------------------------------ NEXT-1 backward reference

def test_backward_ref_is_the_gradient_of_the_forward():
    """backward_ref against the forward reference by central differences
    (the forward is linear in X, A and B, so the difference quotient of a
    scalar loss <dY, Y> is exact up to float64 rounding), and against brute
    force loops on a tiny case."""
    rng = np.random.default_rng(21)
    m, n, k, r, s = 3, 5, 4, 2, 1.5
    x = rng.standard_normal((m, k))
    w = rng.standard_normal((n, k))
    a = rng.standard_normal((r, k))
    b = rng.standard_normal((n, r))
    dy = rng.standard_normal((m, n))
    dx, da, db = oracle.backward_ref(dy, w, x, a, b, s)

    def loss(xx, aa, bb):
        return float(np.sum(dy * oracle.matmul_ref(xx, w, aa, bb, s)))

    h = 1e-3
    for arr, grad in ((x, dx), (a, da), (b, db)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p, q = arr.copy(), arr.copy()
            p[idx] += h
            q[idx] -= h
            args_p = [p if arr is t else t for t in (x, a, b)]
            args_q = [q if arr is t else t for t in (x, a, b)]
            num[idx] = (loss(*args_p) - loss(*args_q)) / (2 * h)
        assert np.allclose(num, grad, rtol=1e-9, atol=1e-9)
    # brute force dX
    bf = np.zeros((m, k))
    for i in range(m):
        for kk in range(k):
            bf[i, kk] = sum(dy[i, j] * w[j, kk] for j in range(n)) + s * sum(
                dy[i, j] * b[j, t] * a[t, kk] for j in range(n) for t in range(r))
    assert np.allclose(bf, dx, rtol=1e-12, atol=1e-12)
    dx0, da0, db0 = oracle.backward_ref(dy, w)
    assert da0 is None and db0 is None and np.allclose(dx0, dy @ w)


# ------------------------------------------- float8 second level (reading C18)

def test_e4m3_values_closed_forms_and_library_decode():
    """Decoding: the landmarks of the format, strict order of the 127
    non-negative finite codes, sign symmetry, and agreement with torch's
    independent float8_e4m3fn conversion for every code."""
    v = np.array([oracle.e4m3_value(c) for c in range(256)])
    assert v[0x00] == 0.0 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6 and v[0x38] == 1.0 and v[0x7E] == 448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.all(np.diff(v[:0x7F]) > 0)
    for c in range(0x7F):
        assert v[c | 0x80] == -v[c]
    torch = pytest.importorskip("torch")
    tv = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ok = ~np.isnan(v)
    assert np.array_equal(np.isnan(tv), np.isnan(v))
    assert np.array_equal(tv[ok], v[ok])


def _e4m3_nearest_exact(x: float) -> int:
    """Brute force over all finite codes with exact rationals, ties to the even code."""
    fx = Fraction(x)
    best = None
    for c in range(0x7F):
        d = abs(abs(fx) - Fraction(oracle.e4m3_value(c)))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (0x80 if x < 0 else 0)


def test_e4m3_encode_brute_force_and_ties():
    rng = np.random.default_rng(18)
    xs = np.concatenate([
        rng.uniform(-448, 448, 300).astype(np.float32),
        (rng.standard_normal(300) * 4).astype(np.float32),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 200).astype(np.float32),   # subnormal range
        np.float32([0.0, 448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -9]),
    ]).astype(np.float32)
    got = oracle.e4m3_encode(xs)
    want = np.array([_e4m3_nearest_exact(float(x)) for x in xs], dtype=np.uint8)
    assert np.array_equal(got, want)
    # every midpoint between neighbouring codes is representable in fp32 and
    # must go to the even code
    mids, even = [], []
    for c in range(0x7E):
        m = (oracle.e4m3_value(c) + oracle.e4m3_value(c + 1)) / 2
        assert float(np.float32(m)) == m
        mids.append(m)
        even.append(c if c % 2 == 0 else c + 1)
    assert np.array_equal(oracle.e4m3_encode(np.float32(mids)), np.array(even, dtype=np.uint8))
    assert np.array_equal(oracle.e4m3_encode(-np.float32(mids)), np.array(even, dtype=np.uint8) | 0x80)
    # round trip of every finite code
    vals = np.float32([oracle.e4m3_value(c) for c in range(0x7F)])
    assert np.array_equal(oracle.e4m3_encode(vals), np.arange(0x7F, dtype=np.uint8))
    torch = pytest.importorskip("torch")
    tq = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got & 0x7F, tq & 0x7F)


def test_e4m3_ratio_table_is_the_rounded_quotient():
    tab = oracle.e4m3_ratio_table()
    for c in range(256):
        v = oracle.e4m3_value(c)
        if v != v:
            assert tab[c] == 0.0
            continue
        assert tab[c] == np.float32(rn32(Fraction(v) / 448))


def test_f8_double_quant_invariants():
    """Each group with s2 > 0 reaches the largest magnitude 448 (codes 0x7E /
    0xFE); every a_hat is within half an E4M3 step (relative 2^-4, or 2^-10
    absolute in the subnormal range, scaled by s2 / 448) plus fp32 roundings
    of the scale; the mean is the exact one of the int8 reading."""
    rng = np.random.default_rng(81)
    a = np.abs(normal_f32((3 * 256 + 17,), 0.02, 81)).astype(np.float32)
    a[5] *= 40.0
    a[300] = 0.0
    q, s2, mean = oracle.double_quant_f8(a)
    _, _, mean_i8 = oracle.double_quant(a)
    assert mean == mean_i8 and q.dtype == np.uint8
    c = (a - mean).astype(np.float32)
    a_hat = oracle.dequant_scales(q, s2, mean, kind="fp8")
    for g in range(s2.size):
        sl = slice(256 * g, min(256 * (g + 1), a.size))
        assert s2[g] == np.abs(c[sl]).max()
        if s2[g] > 0:
            assert np.any((q[sl] & 0x7F) == 0x7E)
        for i in range(sl.start, sl.stop):
            err = abs(float(a_hat[i]) - float(a[i]))
            bound = max(abs(float(c[i])) * 2.0 ** -4, float(s2[g]) / 448 * 2.0 ** -10) + 4e-7 * (abs(float(a[i])) + float(s2[g]))
            assert err <= bound, (i, err, bound)
    # hand check of one value: code 0x38 (1.0) means a_hat = fl32(fl32(s2 / 448) ... ) path
    assert oracle.dequant_scales(np.uint8([0x38]), np.float32([448.0]), np.float32(0.5), kind="fp8")[0] == np.float32(1.5)


def test_dequantize_with_f8_scales_is_the_per_element_product():
    w = normal_f32((3000,), 0.02, 83)
    p, a = oracle.quantize(w)
    q, s2, mean = oracle.double_quant_f8(a)
    got = oracle.dequantize(p, w.size, qabsmax=q, absmax2=s2, mean=mean, dq_kind="fp8")
    a_hat = oracle.dequant_scales(q, s2, mean, kind="fp8")
    codes = oracle.unpack(p, w.size)
    lv = oracle.codebook()
    for i in range(0, w.size, 7):
        assert got[i] == np.float32(rn32(frac(lv[codes[i]]) * frac(a_hat[i // 64])))


# ------------------------------------------------- FP4 code book (READING C19)

def test_e2m1_values_are_the_mx_element_table():
    """The E2M1 element type of the OCP microscaling formats: magnitudes
    0, 0.5, 1, 1.5, 2, 3, 4, 6 for the patterns 000..111, the sign in bit 3."""
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):
        assert oracle.e2m1_value(c) == table[c]
        assert oracle.e2m1_value(c | 8) == -table[c]
    assert math.copysign(1.0, oracle.e2m1_value(8)) == -1.0  # negative zero


def test_fp4_codebook_closed_form_and_symmetry():
    cb = oracle.fp4_codebook()
    assert cb.dtype == np.float32 and cb.shape == (16,)
    for c in range(16):
        assert cb[c] == rn32(Fraction(oracle.e2m1_value(c)).limit_denominator(4) / 6)
    assert cb[7] == np.float32(1.0) and cb[15] == np.float32(-1.0)
    assert cb[0] == 0 and not np.signbit(cb[0]) and cb[8] == 0 and np.signbit(cb[8])
    assert np.array_equal(cb[8:], -cb[:8])
    assert not oracle.FP4_PRODUCED[8] and oracle.FP4_PRODUCED.sum() == 15


def _brute_quantize_fp4(vals):
    a = max(abs(frac(v)) for v in vals)
    af = np.float32(float(a))
    codes = []
    for v in vals:
        q = Fraction(0) if a == 0 else frac(rn32(frac(v) / a))
        codes.append(nearest_level_exact(q, oracle.fp4_codebook()))
    return codes, af


@pytest.mark.parametrize("seed", range(6))
def test_fp4_quantize_matches_brute_force_on_tiny_blocks(seed):
    rng = np.random.default_rng(700 + seed)
    size = int(rng.integers(2, 65))
    kind = ["normal", "uniform", "wide"][seed % 3]
    x = random_blocks_f32(size, 710 + seed, kinds=(kind,))
    packed, absmax = oracle.quantize(x, kind="fp4")
    codes = oracle.unpack(packed, x.size)
    bcodes, ba = _brute_quantize_fp4(list(x))
    assert absmax.shape == (1,) and absmax[0] == ba
    assert list(codes) == bcodes
    assert 8 not in bcodes  # the first of two equally near zeros is the positive one


def test_fp4_levels_round_trip_and_sign_symmetry():
    cb = oracle.fp4_codebook()
    produced = [c for c in range(16) if c != 8]
    for k in (-4, 0, 3):
        s = np.float32(2.0 ** k)
        block = (cb[produced] * s).astype(np.float32)
        packed, absmax = oracle.quantize(block, kind="fp4")
        assert absmax[0] == s
        assert list(oracle.unpack(packed, block.size)) == produced
        deq = oracle.dequantize(packed, block.size, absmax=absmax, kind="fp4")
        assert np.array_equal(deq, block)
    x = random_blocks_f32(640, 720)
    p1, _ = oracle.quantize(x, kind="fp4")
    p2, _ = oracle.quantize(-x, kind="fp4")
    c1, c2 = oracle.unpack(p1, x.size), oracle.unpack(p2, x.size)
    assert np.array_equal(np.where(c1 == 0, 0, c1 ^ 8), c2)


def test_fp4_ties_go_away_from_zero_and_odd_tail_pads_with_zero():
    cb = oracle.fp4_codebook()
    order = sorted((c for c in range(16) if c != 8), key=lambda c: float(cb[c]))
    ties = 0
    for lo, hi in zip(order, order[1:]):
        m = (frac(cb[lo]) + frac(cb[hi])) / 2
        if Fraction(float(rn32(m))) != m:
            continue
        ties += 1
        block = np.array([float(m), 1.0], dtype=np.float32)
        packed, _ = oracle.quantize(block, kind="fp4")
        code = oracle.unpack(packed, 2)[0]
        assert code == (hi if m > 0 else lo)
    assert ties >= 2  # at least the midpoints next to zero
    packed, _ = oracle.quantize(np.array([1.0, -0.5, 0.25], dtype=np.float32), kind="fp4")
    assert packed.size == 2 and packed[1] & 0xF == oracle.FP4_ZERO
