"""Helpers for the GPU parity tests: device fixtures, host<->device copies and
the oracle-side reference for a subset of weight rows."""

from __future__ import annotations

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


def oracle_blocks_dequant_bf16(w_f32: np.ndarray, block_cols, absmax_all: np.ndarray, dq: bool):
    """Oracle bf16 dequantized values of whole 64-column blocks of a weight
    [rows, cols] (cols % 64 == 0): returns [rows, len(block_cols) * 64], the
    blocks in the order given.  Each block quantizes on its own; with double
    quantization its scale comes from the oracle's double_quant over the
    absmax of the whole matrix."""
    rows, cols = w_f32.shape
    bpr = cols // 64
    bc = np.asarray(block_cols, dtype=np.int64)
    sub = np.stack([w_f32[:, 64 * b:64 * b + 64] for b in bc], axis=1)  # [rows, nb, 64]
    packed, absmax = oracle.quantize(np.ascontiguousarray(sub).reshape(-1))
    if dq:
        q, s2, mean = oracle.double_quant(absmax_all)
        a_hat_all = oracle.dequant_scales(q, s2, mean)
        idx = (np.arange(rows, dtype=np.int64)[:, None] * bpr + bc[None, :]).reshape(-1)
        a = a_hat_all[idx]
    else:
        a = absmax
    bits = oracle.dequantize(packed, sub.size, absmax=a, out="bf16")
    return oracle.bf16_bits_to_f32(bits).reshape(rows, len(bc) * 64)
