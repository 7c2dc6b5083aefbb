"""Helpers for the GPU parity tests: device fixtures, host<->device copies and
the oracle-side reference for a subset of weight rows."""

from __future__ import annotations

import functools
import sys

import numpy as np
import pytest

import oracle

# Matmul acceptance bound: relative Frobenius error against the float64
# product of the oracle's bf16-dequantized weights.
MATMUL_RTOL = 1e-2


def say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this container")
    import dequant_matmul_nf4_amd as nf4
    nf4.lib()  # raises if the library is missing: no silent fallback
    return torch


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)) if isinstance(a, np.ndarray) else a
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda").contiguous()


def u8(t):
    return t.cpu().numpy().view(np.uint8)


def bf16_bits(t):
    import torch
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def f32_bits(t):
    return t.cpu().numpy().view(np.uint32)


def oracle_rows_dequant_bf16(w_rows_f32: np.ndarray, row_idx, cols: int, absmax_all: np.ndarray, dq: bool):
    """Oracle bf16 dequantized values of selected weight rows.

    Rows hold whole 64-blocks (cols % 64 == 0), so each row quantizes on its
    own; with double quantization the scales of those rows come from the
    oracle's double_quant over the absmax of the whole matrix."""
    out = np.empty((len(row_idx), cols), dtype=np.float32)
    bpr = cols // 64
    if dq:
        q, s2, mean = oracle.double_quant(absmax_all)
        a_hat_all = oracle.dequant_scales(q, s2, mean)
    for i, r in enumerate(row_idx):
        packed, absmax = oracle.quantize(w_rows_f32[i])
        a = a_hat_all[r * bpr:(r + 1) * bpr] if dq else absmax
        bits = oracle.dequantize(packed, cols, absmax=a, out="bf16")
        out[i] = oracle.bf16_bits_to_f32(bits)
    return out


# ------------------------------------------------ full-size, tile-complete checks
#
# A full-size product is compared with the oracle's float64 product on every
# output.  Three bounds are applied, each chosen so that a plausible kernel
# mistake fails one of them:
#  - relative Frobenius error <= MATMUL_RTOL over the whole output;
#  - the same bound on every output tile (the kernel's own tile shape): a tile
#    that skipped or repeated one K step, or took another tile's operands,
#    is off by several per cent there even when the whole-output norm hides it;
#  - a per-element bound derived from the arithmetic: the output's final
#    rounding (half an ulp of bf16 is at most 2^-8 of the value), the float32
#    accumulation of `terms` products (at most terms * 2^-24 of the sum of
#    their magnitudes, sabs), and the rounding of the weights the kernel takes
#    against those of the reference (w_rel of the same sum).

BF16_HALF_ULP_REL = 2.0 ** -8
F32_EPS = 2.0 ** -24


@functools.lru_cache(maxsize=4)
def oracle_wdeq_full(key: str, out: str = "bf16") -> np.ndarray:
    """The oracle's dequantized weight of a named full-size workload matrix
    (float32 values of the bf16 or float32 dequantized weight), computed once
    per process: quantize, double quant and dequantize of the whole matrix."""
    if key.startswith("c3:"):
        w = bf16_to_f32_np(syn_weight_c3(key[3:]))
    elif key == "c4":
        w = bf16_to_f32_np(syn_c4()["w"])
    else:
        raise KeyError(key)
    p, a = oracle.quantize(w.reshape(-1))
    q, s2, mean = oracle.double_quant(a)
    if out == "bf16":
        bits = oracle.dequantize(p, w.size, qabsmax=q, absmax2=s2, mean=mean, out="bf16")
        return oracle.bf16_bits_to_f32(bits).reshape(w.shape)
    return oracle.dequantize(p, w.size, qabsmax=q, absmax2=s2, mean=mean, out="f32").reshape(w.shape)


def syn_weight_c3(name):
    import synthetic as syn
    return syn.c3_weight(name)


@functools.lru_cache(maxsize=1)
def syn_c4():
    import synthetic as syn
    return syn.c4_inputs()


def bf16_to_f32_np(t) -> np.ndarray:
    import synthetic as syn
    return syn.bf16_to_f32(t)


def tile_rel_frobenius(got: np.ndarray, ref: np.ndarray, tm: int, tn: int):
    """Largest relative Frobenius error over the (tm x tn) tiles of a 2-D
    output (ragged edge tiles included) and the tile where it occurs."""
    M, N = ref.shape
    gm, gn = -(-M // tm), -(-N // tn)
    pad = ((0, gm * tm - M), (0, gn * tn - N))
    d = np.pad(np.asarray(got, np.float64) - ref, pad).reshape(gm, tm, gn, tn)
    r = np.pad(np.asarray(ref, np.float64), pad).reshape(gm, tm, gn, tn)
    num = np.sqrt((d * d).sum(axis=(1, 3)))
    den = np.sqrt((r * r).sum(axis=(1, 3)))
    rel = num / np.where(den > 0, den, 1.0)
    i = np.unravel_index(int(np.argmax(rel)), rel.shape)
    return float(rel[i]), (int(i[0]), int(i[1]))


def check_full_product(got: np.ndarray, ref: np.ndarray, sabs: np.ndarray, terms: int, tile, w_rel: float = 0.0,
                       label: str = ""):
    """The three bounds above; `tile` = (tm, tn) of the kernel's output tiles."""
    got = np.asarray(got, np.float64)
    e = oracle.rel_frobenius(got, ref)
    et, where = tile_rel_frobenius(got, ref, *tile)
    bound = BF16_HALF_ULP_REL * np.abs(ref) + (terms * F32_EPS + w_rel) * sabs + 1e-30
    excess = np.abs(got - ref) / bound
    worst = np.unravel_index(int(np.argmax(excess)), excess.shape)
    say(f"  {label} rel err {e:.2e}; worst tile {et:.2e} at {where}; worst element/bound {excess[worst]:.3f} at "
        f"{tuple(int(v) for v in worst)}")
    assert e <= MATMUL_RTOL, e
    assert et <= MATMUL_RTOL, (et, where)
    assert excess[worst] <= 1.0, (worst, got[worst], ref[worst], bound[worst])
