"""CPU oracle for the NF4 weight path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy code that states what the NF4 path
computes.  Only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import it; the product path (the HIP library and its Python
binding) never does, and the two share no code, tables or constants.

Sources (web pages, cited by title and section; plus the Open Compute
Project's 8-bit floating point specification for the E4M3 format of the
float8 second-level reading and its microscaling (MX) formats specification
for the E2M1 format of the FP4 reading):
  [TOOL]  "bitsandbytes" (ozercemkelahmet.com/tools/bitsandbytes):
          "How it works" Steps 1-5, "How NF4 works", "Double quantization",
          "A worked example", "Memory arithmetic", "Practical guidance and
          best practices".
  [TUT]   "bitsandbytes quantization tutorial: 4-bit and 8-bit models"
          (mljourney.com): "4-bit Loading with NF4", "How NF4 Works",
          "Memory Requirements at Different Precisions", "Merging LoRA
          Adapters After Fine-Tuning".

Readings where the pages leave a step open are marked READING below.

Pins: every function here is pinned by tests/test_oracle_pins.py against
closed forms, exact rational arithmetic, brute force on tiny inputs, library
routines, or the pages' worked example.  No function is parity-unpinned.
"""

from __future__ import annotations

import math
import statistics
from fractions import Fraction

import numpy as np

BLOCKSIZE = 64      # [TOOL] "How it works", Step 1: "for example 64 values at a time"
BLOCKSIZE2 = 256    # second-level block for the quantized scales (READING, see double_quant)

# ------------------------------------------------------------------ code book
#
# [TOOL] "How NF4 works": the 16 code values are placed so that each covers an
# equal share of the bell curve.  [TUT] "How NF4 Works": information-
# theoretically optimal for normally distributed data.  READING: the
# asymmetric equal-probability construction introduced with NF4 (the QLoRA
# paper the tool page names): 8 positive and 7 negative normal quantiles at
# evenly spaced probabilities between delta and 1/2 (1/2 itself excluded),
# plus an exact zero, all divided by the quantile at delta so the ends are
# exactly -1 and +1.  delta = 1 - (1/30 + 1/32)/2 is the mean of the
# outermost bin-centre probabilities for 15 and 16 equal bins.

DELTA = Fraction(1) - (Fraction(1, 30) + Fraction(1, 32)) / 2


def _upper_tail(x: float) -> float:
    """1 - Phi(x) for the standard normal, from the complementary error function."""
    return 0.5 * math.erfc(x / math.sqrt(2.0))


def inv_phi_bisect(p: Fraction) -> float:
    """Phi^{-1}(p) for 1/2 < p < 1 by bisection on the upper tail 1 - Phi(x)."""
    q = float(1 - p)          # tail probability, formed exactly then rounded once
    lo, hi = 0.0, 16.0
    for _ in range(2000):
        mid = 0.5 * (lo + hi)
        if mid == lo or mid == hi:
            break
        if _upper_tail(mid) > q:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def inv_phi_stdlib(p: Fraction) -> float:
    """Phi^{-1}(p) from Python's statistics.NormalDist (an independent routine)."""
    return statistics.NormalDist().inv_cdf(float(p))


def level_probabilities():
    """(positive, negative) probability lists, exact rationals, outermost first."""
    pos = [DELTA + (Fraction(1, 2) - DELTA) * i / 8 for i in range(8)]
    neg = [DELTA + (Fraction(1, 2) - DELTA) * j / 7 for j in range(7)]
    return pos, neg


def levels_f64(inv=inv_phi_bisect) -> np.ndarray:
    """The 16 NF4 levels in float64, ascending (index 0 = -1, 7 = 0, 15 = +1)."""
    pos_p, neg_p = level_probabilities()
    top = inv(DELTA)
    pos = [inv(p) / top for p in pos_p]
    neg = [-inv(p) / top for p in neg_p]
    vals = sorted(neg + [0.0] + pos)
    return np.array(vals, dtype=np.float64)


def codebook() -> np.ndarray:
    """The 16 NF4 levels rounded once to float32, ascending (READING: index order)."""
    return levels_f64().astype(np.float32)


# ------------------------------------------------------- blockwise quantization

def block_absmax(x: np.ndarray, blocksize: int = BLOCKSIZE) -> np.ndarray:
    """[TOOL] "How it works", Steps 1-2: per block, the largest absolute value.

    The last block covers only the elements that exist (READING)."""
    x = np.asarray(x, dtype=np.float32).reshape(-1)
    nb = -(-x.size // blocksize)
    padded = np.zeros(nb * blocksize, dtype=np.float32)
    padded[: x.size] = np.abs(x)
    return padded.reshape(nb, blocksize).max(axis=1)


def nearest_code(v: np.ndarray, levels=None, allowed=None) -> np.ndarray:
    """[TOOL] "How it works", Step 3: index of the nearest code-book entry.

    levels: the code book (default NF4); allowed: the codes that may be
    chosen (default all; the FP4 reading leaves out its negative zero).

    READING: an exact tie between two levels goes to the level farther from
    zero (the only rounding rule the pages state, in "A worked example", rounds
    away from zero).  Distances are taken in float64: the difference of two
    float32 numbers whose exponents differ by at most 29 is exact there, and
    when |v| is too small for that, the zero level wins by a wide margin, so
    the minimum and any tie are decided exactly."""
    lv = (codebook() if levels is None else np.asarray(levels, dtype=np.float32)).astype(np.float64)
    ok = np.ones(lv.size, dtype=bool) if allowed is None else np.asarray(allowed, dtype=bool)
    out = np.empty(v.size, dtype=np.uint8)
    flat = np.asarray(v, dtype=np.float32).reshape(-1)
    step = 1 << 18
    for s in range(0, flat.size, step):
        vv = flat[s : s + step].astype(np.float64)[:, None]
        d = np.where(ok[None, :], np.abs(vv - lv[None, :]), np.inf)
        dmin = d.min(axis=1, keepdims=True)
        tied = d == dmin
        score = np.where(tied, np.abs(lv)[None, :], -1.0)
        out[s : s + step] = score.argmax(axis=1)
    return out


def normalize(x: np.ndarray, absmax: np.ndarray, blocksize: int = BLOCKSIZE) -> np.ndarray:
    """[TOOL] "How it works", Step 2: every value divided by its block's absmax.

    READING: one IEEE float32 division x / a (round to nearest even).  Blocks
    with a = 0 are left at 0."""
    x = np.asarray(x, dtype=np.float32).reshape(-1)
    nb = absmax.size
    padded = np.zeros(nb * blocksize, dtype=np.float32)
    padded[: x.size] = x
    blocks = padded.reshape(nb, blocksize)
    a = np.where(absmax > 0, absmax, np.float32(1.0)).astype(np.float32)
    with np.errstate(over="raise", divide="raise", invalid="raise", under="ignore"):
        out = blocks / a[:, None]
    out[absmax == 0] = 0
    return out.reshape(-1)[: x.size]


def pack(codes: np.ndarray, pad: int = 7) -> np.ndarray:
    """[TOOL] "How it works", Step 4: two 4-bit indices share one byte.

    READING: element 2j in the high nibble, element 2j+1 in the low nibble; an
    odd count is completed with the zero level's index (7 for NF4, 0 for FP4)."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if c.size % 2:
        c = np.concatenate([c, np.array([pad], dtype=np.uint8)])
    return ((c[0::2] << 4) | c[1::2]).astype(np.uint8)


def unpack(packed: np.ndarray, n: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    c = np.empty(2 * p.size, dtype=np.uint8)
    c[0::2] = p >> 4
    c[1::2] = p & 0xF
    return c[:n]


def quantize(x: np.ndarray, blocksize: int = BLOCKSIZE, kind: str = "nf4"):
    """Steps 1-4: returns (packed uint8 [ceil(n/2)], absmax float32 [ceil(n/64)]).

    Inputs are float32 values (bf16 inputs are passed as their exact float32
    widening).  kind="fp4" uses the FP4 code book (READING C19 below)."""
    x = np.asarray(x, dtype=np.float32).reshape(-1)
    absmax = block_absmax(x, blocksize)
    if kind == "fp4":
        codes = nearest_code(normalize(x, absmax, blocksize), fp4_codebook(), FP4_PRODUCED)
        return pack(codes, pad=FP4_ZERO), absmax
    if kind != "nf4":
        raise ValueError(kind)
    codes = nearest_code(normalize(x, absmax, blocksize))
    return pack(codes), absmax


# ------------------------------------------------- FP4 code book (READING C19)
#
# [TOOL] "What it is" lists FP4 beside NF4 among the 4-bit formats of the
# quantized linear layers and its "Glossary" calls FP4 a 4-bit floating-point
# data type; the page "Environment: Huggingface Transformers BitsAndBytes
# Quantization Env" ("Description") names NF4/FP4 as the two 4-bit choices.
# No values are given.  READING: the 4-bit float is the E2M1 element type of
# the Open Compute Project's microscaling (MX) formats specification -- a sign
# bit, two exponent bits with bias 1 and one mantissa bit, exponent field 0
# subnormal (value m / 2) -- so the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.
# The code book ("Glossary": the table of allowed values that indices point
# to) is those values divided by 6, so that the block absmax maps to +-1 as
# NF4's outermost levels do.  A code is the 4-bit pattern itself (sign in bit
# 3).  Pattern 1000 (negative zero) decodes to -0 and is never produced:
# quantization chooses among the other 15 codes, zero going to 0000, with the
# same nearest rule (ties to the level farther from zero).  Everything else
# (absmax per 64, normalisation, packing, double quantization, the consumers)
# is the NF4 path with this code book.

FP4_ZERO = 0
FP4_PRODUCED = np.array([c != 8 for c in range(16)])


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 pattern (sign, 2 exponent bits with bias 1, 1 mantissa bit)."""
    sign = -1.0 if code & 8 else 1.0
    e, m = (code >> 1) & 3, code & 1
    mag = m / 2 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
    return sign * mag


def fp4_codebook() -> np.ndarray:
    """The 16 FP4 levels by code: e2m1_value(code) / 6 rounded once to float32."""
    return np.array([e2m1_value(c) / 6.0 for c in range(16)], dtype=np.float32)


# --------------------------------------------------------- double quantization
#
# [TOOL] "Double quantization" and [TUT] "4-bit Loading with NF4": the per-block
# scales are quantized again.  READING: the scales are centred on their mean
# and quantized to int8 in blocks of 256 with the linear absmax scheme of
# [TOOL] "A worked example" (scale by 127, round half away from zero; dequantize
# by dividing by 127 and multiplying by the block's absmax).  [TUT] "How NF4
# Works" says float8; the int8 reading is the one used here.

def int8_absmax_quantize(v: np.ndarray, blocksize: int):
    """[TOOL] "A worked example": linear int8 absmax quantization per block.

    t = fl32(fl32(v / s) * 127), q = sign(t) * floor(|t| + 1/2); s = the block's
    largest |v|; a block with s = 0 gets q = 0.  Returns (q int8, s float32)."""
    v = np.asarray(v, dtype=np.float32).reshape(-1)
    nb = -(-v.size // blocksize)
    padded = np.zeros(nb * blocksize, dtype=np.float32)
    padded[: v.size] = v
    blocks = padded.reshape(nb, blocksize)
    s = np.abs(blocks).max(axis=1).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    with np.errstate(under="ignore"):
        t = (blocks / safe[:, None]).astype(np.float32) * np.float32(127.0)
    t = t.astype(np.float32)
    t64 = t.astype(np.float64)                      # exact widening
    q = np.sign(t64) * np.floor(np.abs(t64) + 0.5)  # exact: |t| <= 127
    q = np.clip(q, -127, 127)
    q[s == 0] = 0
    return q.reshape(-1)[: v.size].astype(np.int8), s


def exact_mean_f32(a: np.ndarray) -> np.float32:
    """Mean of the scales: the exact sum rounded once to float64 (math.fsum),
    divided by the count in float64, rounded to float32 (READING)."""
    a = np.asarray(a, dtype=np.float32).reshape(-1)
    total = math.fsum(a.astype(np.float64).tolist())
    return np.float32(total / a.size)


def double_quant(absmax: np.ndarray, blocksize2: int = BLOCKSIZE2):
    """Returns (qabsmax int8 [nb], absmax2 float32 [ceil(nb/256)], mean float32)."""
    a = np.asarray(absmax, dtype=np.float32).reshape(-1)
    mean = exact_mean_f32(a)
    centred = (a - mean).astype(np.float32)
    q, s2 = int8_absmax_quantize(centred, blocksize2)
    return q, s2, mean


def dequant_scales(q: np.ndarray, absmax2: np.ndarray, mean, blocksize2: int = BLOCKSIZE2,
                   kind: str = "int8") -> np.ndarray:
    """a_hat = fl32(fl32(fl32(q / 127) * s2) + mean): [TOOL] "A worked example"
    (divide by 127, multiply by the scale) followed by adding the mean back.
    kind="fp8": the first factor is fl32(e4m3(q) / 448) instead (see below)."""
    s2 = np.asarray(absmax2, dtype=np.float32).reshape(-1)
    if kind == "fp8":
        codes = np.asarray(q).reshape(-1).view(np.uint8) if np.asarray(q).dtype != np.uint8 else np.asarray(q).reshape(-1)
        t = e4m3_ratio_table()[codes.astype(np.int64)]
    else:
        q = np.asarray(q, dtype=np.int8).reshape(-1)
        t = (q.astype(np.float32) / np.float32(127.0)).astype(np.float32)
    g = np.arange(t.size) // blocksize2
    t = (t * s2[g]).astype(np.float32)
    return (t + np.float32(mean)).astype(np.float32)


# ------------------------------------------- float8 second level (READING C18)
#
# [TUT] "How NF4 Works" says the scales go from float32 to float8.  The pages
# name no 8-bit float format; the reading here is E4M3 as defined in the Open
# Compute Project's 8-bit floating point specification (OFP8): 1 sign bit, 4
# exponent bits with bias 7, 3 mantissa bits, subnormals, no infinities, the
# all-ones exponent and mantissa pattern is NaN, largest finite value 448.
# The step mirrors the int8 one: t = fl32(fl32(c / s2) * 448), the code is
# the E4M3 value nearest to t (ties to the even mantissa), and dequantization
# multiplies fl32(e4m3(q) / 448) by s2 and adds the mean back.

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """The value of an E4M3 code (NaN for the two NaN patterns)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9          # subnormal: m/8 * 2^(1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_encode(t: np.ndarray) -> np.ndarray:
    """E4M3 code nearest to each float32 t with |t| <= 448, ties to the even
    mantissa; the sign of t is kept (t = +0 gives code 0)."""
    t = np.asarray(t, dtype=np.float32).reshape(-1)
    finite = [(e4m3_value(c), c) for c in range(0x7F)]          # +0 .. 448, ascending
    mags = np.array([v for v, _ in finite], dtype=np.float64)
    out = np.empty(t.size, dtype=np.uint8)
    for i, x in enumerate(t.astype(np.float64)):
        a = abs(x)
        if not a <= E4M3_MAX:
            raise ValueError("e4m3_encode: |t| out of range")
        k = int(np.searchsorted(mags, a))            # mags[k - 1] < a <= mags[k]
        if k < mags.size and mags[k] == a:
            c = k
        else:
            lo, hi = k - 1, k
            dlo, dhi = a - mags[lo], mags[hi] - a
            if dlo < dhi:
                c = lo
            elif dhi < dlo:
                c = hi
            else:
                c = lo if (lo & 1) == 0 else hi     # even mantissa (codes alternate parity)
        out[i] = c | (0x80 if x < 0 else 0)
    return out


def e4m3_ratio_table() -> np.ndarray:
    """fl32(e4m3(q) / 448) for every code q (0 for the NaN codes, never produced)."""
    tab = np.zeros(256, dtype=np.float32)
    for c in range(256):
        v = e4m3_value(c)
        if v == v:
            tab[c] = np.float32(v) / np.float32(E4M3_MAX)
    return tab


def f8_absmax_quantize(v: np.ndarray, blocksize: int):
    """The float8 reading of the second level: per block s = max |v|,
    t = fl32(fl32(v / s) * 448), q = e4m3_encode(t); s = 0 gives code 0.
    Returns (q uint8, s float32)."""
    v = np.asarray(v, dtype=np.float32).reshape(-1)
    nb = -(-v.size // blocksize)
    padded = np.zeros(nb * blocksize, dtype=np.float32)
    padded[: v.size] = v
    blocks = padded.reshape(nb, blocksize)
    s = np.abs(blocks).max(axis=1).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    with np.errstate(under="ignore"):
        t = (blocks / safe[:, None]).astype(np.float32) * np.float32(E4M3_MAX)
    t = t.astype(np.float32)
    t[s == 0] = 0.0
    q = e4m3_encode(t.reshape(-1)).reshape(nb, blocksize)
    return q.reshape(-1)[: v.size], s


def double_quant_f8(absmax: np.ndarray, blocksize2: int = BLOCKSIZE2):
    """Returns (qabsmax uint8 E4M3 codes [nb], absmax2 float32 [ceil(nb/256)], mean float32)."""
    a = np.asarray(absmax, dtype=np.float32).reshape(-1)
    mean = exact_mean_f32(a)
    centred = (a - mean).astype(np.float32)
    q, s2 = f8_absmax_quantize(centred, blocksize2)
    return q, s2, mean


# ------------------------------------------------------------- dequantization

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16 bit patterns (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def dequantize(packed, n: int, absmax=None, qabsmax=None, absmax2=None, mean=None,
               blocksize: int = BLOCKSIZE, blocksize2: int = BLOCKSIZE2, out: str = "f32", dq_kind: str = "int8",
               kind: str = "nf4"):
    """[TOOL] "How it works", Step 5: expand each code with its block's scale.

    w = fl32(level[code] * a_hat); for out="bf16" the float32 value is rounded
    once to nearest even and the bf16 bit patterns (uint16) are returned.
    dq_kind selects the second level's reading (int8 or fp8), kind the code
    book (nf4 or fp4)."""
    codes = unpack(packed, n)
    lv = fp4_codebook() if kind == "fp4" else codebook()
    if absmax is not None:
        a_hat = np.asarray(absmax, dtype=np.float32).reshape(-1)
    else:
        a_hat = dequant_scales(qabsmax, absmax2, mean, blocksize2, kind=dq_kind)
    blk = np.arange(n) // blocksize
    w = (lv[codes] * a_hat[blk]).astype(np.float32)
    if out == "f32":
        return w
    if out == "bf16":
        return f32_to_bf16_bits(w)
    raise ValueError(out)


# -------------------------------------------------------------- matmul reference

def matmul_ref(x: np.ndarray, w_deq: np.ndarray, lora_a=None, lora_b=None, lora_scale: float = 0.0):
    """Y = X . W^T (+ s . (X . A^T) . B^T), all in float64.

    x: [M, K] values, w_deq: [N, K] dequantized weights, lora_a: [r, K],
    lora_b: [N, r].  [TOOL] "How it works", Step 5 (dequantize then multiply);
    [TUT] "QLoRA: Fine-Tuning a 4-bit Model" (adapters on the frozen base, the
    adapter output multiplied by a scale factor)."""
    x64 = np.asarray(x, dtype=np.float64)
    w64 = np.asarray(w_deq, dtype=np.float64)
    y = x64 @ w64.T
    if lora_a is not None:
        t = x64 @ np.asarray(lora_a, dtype=np.float64).T
        y = y + float(lora_scale) * (t @ np.asarray(lora_b, dtype=np.float64).T)
    return y


def backward_ref(dy: np.ndarray, w_deq: np.ndarray, x=None, lora_a=None, lora_b=None, lora_scale: float = 0.0):
    """Gradients of Y = X . W^T + s . (X . A^T) . B^T with the base W frozen,
    all in float64 ([TUT] "QLoRA: Fine-Tuning a 4-bit Model": the 4-bit base
    stays frozen and the gradients flow through it to the adapters):

        dX = dY . W + s . (dY . B) . A
        dA = s . (dY . B)^T . X        dB = s . dY^T . (X . A^T)

    dy: [M, N], w_deq: [N, K], x: [M, K], lora_a: [r, K], lora_b: [N, r].
    Returns dX, and (dA, dB) when the adapters are given."""
    dy64 = np.asarray(dy, dtype=np.float64)
    dx = dy64 @ np.asarray(w_deq, dtype=np.float64)
    if lora_a is None:
        return dx, None, None
    a64 = np.asarray(lora_a, dtype=np.float64)
    b64 = np.asarray(lora_b, dtype=np.float64)
    u = float(lora_scale) * (dy64 @ b64)
    dx = dx + u @ a64
    da = db = None
    if x is not None:
        x64 = np.asarray(x, dtype=np.float64)
        da = u.T @ x64
        db = float(lora_scale) * (dy64.T @ (x64 @ a64.T))
    return dx, da, db


def rel_frobenius(y, y_ref) -> float:
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref)
    return float(np.linalg.norm(y - y_ref) / den) if den > 0 else float(np.linalg.norm(y))


# ------------------------------------------------------------------ LoRA merge

def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns, one rounding to nearest even (finite
    inputs).  Method: round to odd into float32 (24 significant bits, at least
    two more than bfloat16's 8 and the same exponent range), then round to
    nearest even into bfloat16; rounding to odd first makes the two steps
    equal one correct rounding."""
    v = np.asarray(v, dtype=np.float64)
    f = v.astype(np.float32)
    back = f.astype(np.float64)
    u = f.view(np.uint32).copy()
    inexact = back != v
    away = inexact & (np.abs(back) > np.abs(v))  # rounded away from zero: step back one ulp
    u[away] -= np.uint32(1)
    u[inexact] |= np.uint32(1)
    return f32_to_bf16_bits(u.view(np.float32))


def f64_to_f16_bits(v: np.ndarray) -> np.ndarray:
    """float64 -> IEEE binary16 bit patterns, one rounding to nearest even,
    subnormals included (numpy's double-to-half conversion rounds once)."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def lora_merge(w_deq_f32: np.ndarray, lora_a: np.ndarray, lora_b: np.ndarray, lora_scale: float,
               out: str = "bf16") -> np.ndarray:
    """[TUT] "Merging LoRA Adapters After Fine-Tuning": after training, the
    adapters are folded into one dense 16-bit copy of the base, which first
    needs the base dequantized ([TOOL] "Practical guidance and best
    practices": merging adds another rounding step).

        W'[n][k] = round( deq[n][k] + s * sum_j B[n][j] * A[j][k] )

    w_deq_f32: [N, K] float32 dequantized base (as dequantize(..., "f32"));
    lora_a: [r, K], lora_b: [N, r] (bf16 values as float32); s = lora_scale
    as float32.  READING: the sum is formed in float64 with j ascending (each
    bf16 x bf16 product is exact in float64, and so is the sum unless its
    terms span more than about 37 binary orders), multiplied by s, added to
    deq in float64, then rounded once to nearest even into out ("bf16" or
    "f16"; the tutorial's merged checkpoint is float16).  Returns uint16 bit
    patterns."""
    deq = np.asarray(w_deq_f32, dtype=np.float32).astype(np.float64)
    a = np.asarray(lora_a, dtype=np.float32).astype(np.float64)
    b = np.asarray(lora_b, dtype=np.float32).astype(np.float64)
    acc = np.zeros(deq.shape, dtype=np.float64)
    for j in range(a.shape[0]):
        acc = acc + b[:, j:j + 1] * a[j:j + 1, :]
    v = deq + np.float64(np.float32(lora_scale)) * acc
    if out == "bf16":
        return f64_to_bf16_bits(v)
    if out == "f16":
        return f64_to_f16_bits(v)
    raise ValueError(out)


# ------------------------------------------------------------ storage footprint

def storage_bytes(n: int, double_quant: bool, blocksize: int = BLOCKSIZE, blocksize2: int = BLOCKSIZE2) -> dict:
    """Bytes of each stored array for n weights ([TOOL] "How it works", Step 4:
    packed indices with the scales stored beside them)."""
    nb = -(-n // blocksize)
    out = {"packed": -(-n // 2)}
    if double_quant:
        out.update(qabsmax=nb, absmax2=4 * (-(-nb // blocksize2)), mean=4)
    else:
        out.update(absmax=4 * nb)
    return out


def bits_per_param(n: int, double_quant: bool) -> float:
    return 8.0 * sum(storage_bytes(n, double_quant).values()) / n
