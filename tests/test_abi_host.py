"""Host-only checks of the C ABI (no GPU needed): the library loads, exports
every function include/nf4.h declares, derives the same code book as the
oracle, and rejects bad arguments before touching the device."""

from __future__ import annotations

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import dequant_matmul_nf4_amd as nf4
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nf4.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nf4.LIB_PATH):
        from dequant_matmul_nf4_amd import build
        build.build()
    return nf4.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nf4_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_expected_calls():
    assert declared_functions() == sorted(nf4.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", nf4.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (nf4_[a-z_0-9]+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_codebook_bit_identical_to_oracle(L):
    cb = np.array(nf4.nf4_codebook(), dtype=np.float32)
    assert np.array_equal(cb.view(np.uint32), oracle.codebook().view(np.uint32))


def test_e4m3_ratio_bit_identical_to_oracle(L):
    """The float8 second level's table (built at compile time in the library)
    against the oracle's, which is pinned to exact rational quotients."""
    tab = np.array(nf4.nf4_e4m3_ratio(), dtype=np.float32)
    assert np.array_equal(tab.view(np.uint32), oracle.e4m3_ratio_table().view(np.uint32))


def test_workspace_sizes(L):
    assert nf4.nf4_double_quant_workspace(1) >= 16 * 8
    assert nf4.nf4_double_quant_workspace(1 << 30) <= WS
    assert nf4.nf4_gemm_workspace(4096, 14336, 0) == 0
    assert nf4.nf4_gemm_workspace(4096, 14336, 16) >= 4096 * 32 * 2
    assert nf4.nf4_gemm_workspace(4096, 14336, 16) % 256 == 0
    assert nf4.nf4_gemm_dx_workspace(4096, 14336, 0) == 0
    # U (m x 2 r_pad bf16, rounded up to 64) and B transposed (r x rows bf16)
    assert nf4.nf4_gemm_dx_workspace(4096, 14336, 16) >= (4096 * 64 + 16 * 14336) * 2
    assert nf4.nf4_gemm_dx_workspace(4096, 14336, 16) % 256 == 0


def test_struct_layout():
    assert ctypes.sizeof(nf4.nf4_weight) == 80
    assert nf4.nf4_weight.blocksize2.offset == 64
    assert nf4.nf4_weight.dq_type.offset == 68
    assert nf4.nf4_weight.quant_type.offset == 72


# Fake but aligned device addresses: every call below fails validation on the
# host, before any HIP call, so nothing is dereferenced.
A = 0x10000
A2 = 0x20000
WS = 1 << 20   # a workspace size larger than any call needs


def _w(**kw):
    base = dict(packed=A, rows=16, cols=64, blocksize=64, absmax=A2, qabsmax=None, absmax2=None, mean=None, blocksize2=256)
    base.update(kw)
    return nf4.nf4_weight(**base)


CASES = [
    ("quantize null x", lambda L: L.nf4_quantize(None, 1, 64, 64, A, A2, None), nf4.NF4_ERR_NULL),
    ("quantize null packed", lambda L: L.nf4_quantize(A, 1, 64, 64, None, A2, None), nf4.NF4_ERR_NULL),
    ("quantize bad dtype", lambda L: L.nf4_quantize(A, 7, 64, 64, A, A2, None), nf4.NF4_ERR_DTYPE),
    ("quantize n=0", lambda L: L.nf4_quantize(A, 1, 0, 64, A, A2, None), nf4.NF4_ERR_SIZE),
    ("quantize n<0", lambda L: L.nf4_quantize(A, 1, -5, 64, A, A2, None), nf4.NF4_ERR_SIZE),
    ("quantize blocksize", lambda L: L.nf4_quantize(A, 1, 64, 128, A, A2, None), nf4.NF4_ERR_BLOCKSIZE),
    ("quantize misaligned x", lambda L: L.nf4_quantize(A + 2, 1, 64, 64, A, A2, None), nf4.NF4_ERR_ALIGN),
    ("quantize misaligned packed", lambda L: L.nf4_quantize(A, 1, 64, 64, A + 8, A2, None), nf4.NF4_ERR_ALIGN),
    ("quantize misaligned absmax", lambda L: L.nf4_quantize(A, 1, 64, 64, A, A2 + 2, None), nf4.NF4_ERR_ALIGN),
    ("dq null", lambda L: L.nf4_double_quant(A, 10, 256, None, A2, A2, A, WS, None), nf4.NF4_ERR_NULL),
    ("dq nblocks", lambda L: L.nf4_double_quant(A, 0, 256, A, A2, A2, A, WS, None), nf4.NF4_ERR_SIZE),
    ("dq blocksize2", lambda L: L.nf4_double_quant(A, 10, 128, A, A2, A2, A, WS, None), nf4.NF4_ERR_BLOCKSIZE),
    ("dq workspace small", lambda L: L.nf4_double_quant(A, 10, 256, A, A2, A2, A, 8, None), nf4.NF4_ERR_WORKSPACE),
    ("dq workspace null", lambda L: L.nf4_double_quant(A, 10, 256, A, A2, A2, None, WS, None), nf4.NF4_ERR_WORKSPACE),
    ("dq misaligned q", lambda L: L.nf4_double_quant(A, 10, 256, A + 1, A2, A2, A, WS, None), nf4.NF4_ERR_ALIGN),
    ("dq noalloc null", lambda L: L.nf4_double_quant_noalloc(A, 10, 256, None, A2, A2, None), nf4.NF4_ERR_NULL),
    ("dq noalloc nblocks 0", lambda L: L.nf4_double_quant_noalloc(A, 0, 256, A, A2, A2, None), nf4.NF4_ERR_SIZE),
    ("dq noalloc nblocks 2^31", lambda L: L.nf4_double_quant_noalloc(A, 1 << 31, 256, A, A2, A2, None), nf4.NF4_ERR_SIZE),
    ("dq noalloc blocksize2", lambda L: L.nf4_double_quant_noalloc(A, 10, 128, A, A2, A2, None), nf4.NF4_ERR_BLOCKSIZE),
    ("dq noalloc misaligned absmax", lambda L: L.nf4_double_quant_noalloc(A + 4, 10, 256, A, A2, A2, None), nf4.NF4_ERR_ALIGN),
    ("dq noalloc misaligned mean", lambda L: L.nf4_double_quant_noalloc(A, 10, 256, A, A2, A2 + 2, None), nf4.NF4_ERR_ALIGN),
    ("dq f8 null", lambda L: L.nf4_double_quant_f8(A, 10, 256, None, A2, A2, A, WS, None), nf4.NF4_ERR_NULL),
    ("dq f8 blocksize2", lambda L: L.nf4_double_quant_f8(A, 10, 128, A, A2, A2, A, WS, None), nf4.NF4_ERR_BLOCKSIZE),
    ("dq f8 workspace small", lambda L: L.nf4_double_quant_f8(A, 10, 256, A, A2, A2, A, 8, None), nf4.NF4_ERR_WORKSPACE),
    ("dequant dq_type unknown", lambda L: L.nf4_dequantize(ctypes.byref(_w(absmax=None, qabsmax=A, absmax2=A2, mean=A2, dq_type=2)), A, 1, None), nf4.NF4_ERR_DTYPE),
    ("dequant quant_type unknown", lambda L: L.nf4_dequantize(ctypes.byref(_w(quant_type=2)), A, 1, None), nf4.NF4_ERR_DTYPE),
    ("gemv quant_type unknown", lambda L: L.nf4_gemv(ctypes.byref(_w(absmax=None, qabsmax=A, absmax2=A2, mean=A2, quant_type=-1)), A, 1, A, 1, None), nf4.NF4_ERR_DTYPE),
    ("quantize_fp4 null", lambda L: L.nf4_quantize_fp4(None, 1, 64, 64, A, A, None), nf4.NF4_ERR_NULL),
    ("quantize_fp4 blocksize", lambda L: L.nf4_quantize_fp4(A, 1, 64, 32, A, A, None), nf4.NF4_ERR_BLOCKSIZE),
    ("gemv dq_type unknown", lambda L: L.nf4_gemv(ctypes.byref(_w(absmax=None, qabsmax=A, absmax2=A2, mean=A2, dq_type=-1)), A, 1, A, 1, None), nf4.NF4_ERR_DTYPE),
    ("e4m3 ratio null", lambda L: L.nf4_e4m3_ratio(None), nf4.NF4_ERR_NULL),
    ("dequant null weight", lambda L: L.nf4_dequantize(None, A, 1, None), nf4.NF4_ERR_NULL),
    ("dequant null out", lambda L: L.nf4_dequantize(ctypes.byref(_w()), None, 1, None), nf4.NF4_ERR_NULL),
    ("dequant bad dtype", lambda L: L.nf4_dequantize(ctypes.byref(_w()), A, 3, None), nf4.NF4_ERR_DTYPE),
    ("dequant blocksize", lambda L: L.nf4_dequantize(ctypes.byref(_w(blocksize=32)), A, 1, None), nf4.NF4_ERR_BLOCKSIZE),
    ("dequant shape", lambda L: L.nf4_dequantize(ctypes.byref(_w(rows=0)), A, 1, None), nf4.NF4_ERR_SIZE),
    ("dequant dq missing", lambda L: L.nf4_dequantize(ctypes.byref(_w(absmax=None)), A, 1, None), nf4.NF4_ERR_NULL),
    ("dequant blocksize2", lambda L: L.nf4_dequantize(ctypes.byref(_w(absmax=None, qabsmax=A, absmax2=A2, mean=A2, blocksize2=64)), A, 1, None), nf4.NF4_ERR_BLOCKSIZE),
    ("dequant misaligned out", lambda L: L.nf4_dequantize(ctypes.byref(_w()), A + 4, 1, None), nf4.NF4_ERR_ALIGN),
    ("dequant misaligned packed", lambda L: L.nf4_dequantize(ctypes.byref(_w(packed=A + 1)), A, 1, None), nf4.NF4_ERR_ALIGN),
    ("gemv cols%64", lambda L: L.nf4_gemv(ctypes.byref(_w(cols=96)), A, 1, A, 1, None), nf4.NF4_ERR_SIZE),
    ("gemv m=0", lambda L: L.nf4_gemv(ctypes.byref(_w()), A, 0, A, 1, None), nf4.NF4_ERR_SIZE),
    ("gemv m=17", lambda L: L.nf4_gemv(ctypes.byref(_w()), A, 17, A, 1, None), nf4.NF4_ERR_SIZE),
    ("gemv null y", lambda L: L.nf4_gemv(ctypes.byref(_w()), A, 1, None, 1, None), nf4.NF4_ERR_NULL),
    ("gemv bad dtype", lambda L: L.nf4_gemv(ctypes.byref(_w()), A, 1, A, 9, None), nf4.NF4_ERR_DTYPE),
    ("gemv misaligned x", lambda L: L.nf4_gemv(ctypes.byref(_w()), A + 2, 1, A, 1, None), nf4.NF4_ERR_ALIGN),
    ("gemm cols%64", lambda L: L.nf4_gemm(ctypes.byref(_w(cols=100)), A, 4, A, None, None, 0, 0.0, None, 0, None), nf4.NF4_ERR_SIZE),
    ("gemm m=0", lambda L: L.nf4_gemm(ctypes.byref(_w()), A, 0, A, None, None, 0, 0.0, None, 0, None), nf4.NF4_ERR_SIZE),
    ("gemm half lora", lambda L: L.nf4_gemm(ctypes.byref(_w()), A, 4, A, A, None, 16, 2.0, A, 4096, None), nf4.NF4_ERR_NULL),
    ("gemm rank 0", lambda L: L.nf4_gemm(ctypes.byref(_w()), A, 4, A, A, A, 0, 2.0, A, 4096, None), nf4.NF4_ERR_SIZE),
    ("gemm rank 65", lambda L: L.nf4_gemm(ctypes.byref(_w()), A, 4, A, A, A, 65, 2.0, A, 1 << 20, None), nf4.NF4_ERR_SIZE),
    ("gemm r without lora", lambda L: L.nf4_gemm(ctypes.byref(_w()), A, 4, A, None, None, 3, 0.0, None, 0, None), nf4.NF4_ERR_SIZE),
    ("gemm workspace small", lambda L: L.nf4_gemm(ctypes.byref(_w()), A, 4, A, A, A, 16, 2.0, A, 16, None), nf4.NF4_ERR_WORKSPACE),
    ("gemm workspace null", lambda L: L.nf4_gemm(ctypes.byref(_w()), A, 4, A, A, A, 16, 2.0, None, 4096, None), nf4.NF4_ERR_WORKSPACE),
    ("gemm scale nan", lambda L: L.nf4_gemm(ctypes.byref(_w()), A, 4, A, A, A, 16, float("nan"), A, 4096, None), nf4.NF4_ERR_SIZE),
    ("gemm misaligned y", lambda L: L.nf4_gemm(ctypes.byref(_w()), A, 4, A + 2, None, None, 0, 0.0, None, 0, None), nf4.NF4_ERR_ALIGN),
    ("dx null weight", lambda L: L.nf4_gemm_dx(None, A, 4, A, None, None, 0, 0.0, None, 0, None), nf4.NF4_ERR_NULL),
    ("dx null dy", lambda L: L.nf4_gemm_dx(ctypes.byref(_w()), None, 4, A, None, None, 0, 0.0, None, 0, None), nf4.NF4_ERR_NULL),
    ("dx null dx", lambda L: L.nf4_gemm_dx(ctypes.byref(_w()), A, 4, None, None, None, 0, 0.0, None, 0, None), nf4.NF4_ERR_NULL),
    ("dx cols%64", lambda L: L.nf4_gemm_dx(ctypes.byref(_w(cols=96)), A, 4, A, None, None, 0, 0.0, None, 0, None), nf4.NF4_ERR_SIZE),
    ("dx rows%8", lambda L: L.nf4_gemm_dx(ctypes.byref(_w(rows=12)), A, 4, A, None, None, 0, 0.0, None, 0, None), nf4.NF4_ERR_SIZE),
    ("dx m=0", lambda L: L.nf4_gemm_dx(ctypes.byref(_w()), A, 0, A, None, None, 0, 0.0, None, 0, None), nf4.NF4_ERR_SIZE),
    ("dx half lora", lambda L: L.nf4_gemm_dx(ctypes.byref(_w()), A, 4, A, None, A, 16, 2.0, A, WS, None), nf4.NF4_ERR_NULL),
    ("dx rank 65", lambda L: L.nf4_gemm_dx(ctypes.byref(_w()), A, 4, A, A, A, 65, 2.0, A, WS, None), nf4.NF4_ERR_SIZE),
    ("dx r without lora", lambda L: L.nf4_gemm_dx(ctypes.byref(_w()), A, 4, A, None, None, 2, 0.0, None, 0, None), nf4.NF4_ERR_SIZE),
    ("dx scale inf", lambda L: L.nf4_gemm_dx(ctypes.byref(_w()), A, 4, A, A, A, 16, float("-inf"), A, WS, None), nf4.NF4_ERR_SIZE),
    ("dx workspace small", lambda L: L.nf4_gemm_dx(ctypes.byref(_w()), A, 4, A, A, A, 16, 2.0, A, 64, None), nf4.NF4_ERR_WORKSPACE),
    ("dx workspace null", lambda L: L.nf4_gemm_dx(ctypes.byref(_w()), A, 4, A, A, A, 16, 2.0, None, WS, None), nf4.NF4_ERR_WORKSPACE),
    ("dx misaligned workspace", lambda L: L.nf4_gemm_dx(ctypes.byref(_w()), A, 4, A, A, A, 16, 2.0, A + 16, WS, None), nf4.NF4_ERR_ALIGN),
    ("dx misaligned dy", lambda L: L.nf4_gemm_dx(ctypes.byref(_w()), A + 2, 4, A, None, None, 0, 0.0, None, 0, None), nf4.NF4_ERR_ALIGN),
    ("dx misaligned a", lambda L: L.nf4_gemm_dx(ctypes.byref(_w()), A, 4, A, A + 8, A, 16, 2.0, A, WS, None), nf4.NF4_ERR_ALIGN),
    ("grads null x", lambda L: L.nf4_lora_grads(None, A, 4, 64, 64, A, A, 16, 2.0, A, A, A, WS, None), nf4.NF4_ERR_NULL),
    ("grads null b", lambda L: L.nf4_lora_grads(A, A, 4, 64, 64, A, None, 16, 2.0, A, A, A, WS, None), nf4.NF4_ERR_NULL),
    ("grads no outputs", lambda L: L.nf4_lora_grads(A, A, 4, 64, 64, A, A, 16, 2.0, None, None, A, WS, None), nf4.NF4_ERR_NULL),
    ("grads m=0", lambda L: L.nf4_lora_grads(A, A, 0, 64, 64, A, A, 16, 2.0, A, A, A, WS, None), nf4.NF4_ERR_SIZE),
    ("grads rows%8", lambda L: L.nf4_lora_grads(A, A, 4, 60, 64, A, A, 16, 2.0, A, A, A, WS, None), nf4.NF4_ERR_SIZE),
    ("grads cols%8", lambda L: L.nf4_lora_grads(A, A, 4, 64, 68, A, A, 16, 2.0, A, A, A, WS, None), nf4.NF4_ERR_SIZE),
    ("grads rank 0", lambda L: L.nf4_lora_grads(A, A, 4, 64, 64, A, A, 0, 2.0, A, A, A, WS, None), nf4.NF4_ERR_SIZE),
    ("grads scale nan", lambda L: L.nf4_lora_grads(A, A, 4, 64, 64, A, A, 16, float("nan"), A, A, A, WS, None), nf4.NF4_ERR_SIZE),
    ("grads misaligned da", lambda L: L.nf4_lora_grads(A, A, 4, 64, 64, A, A, 16, 2.0, A + 4, A, A, WS, None), nf4.NF4_ERR_ALIGN),
    ("grads workspace small", lambda L: L.nf4_lora_grads(A, A, 4, 64, 64, A, A, 16, 2.0, A, A, A, 64, None), nf4.NF4_ERR_WORKSPACE),
    ("grads misaligned workspace", lambda L: L.nf4_lora_grads(A, A, 4, 64, 64, A, A, 16, 2.0, A, A, A + 128, WS, None), nf4.NF4_ERR_ALIGN),
    ("merge null weight", lambda L: L.nf4_lora_merge(None, A, A, 16, 2.0, A, 1, None), nf4.NF4_ERR_NULL),
    ("merge null a", lambda L: L.nf4_lora_merge(ctypes.byref(_w()), None, A, 16, 2.0, A, 1, None), nf4.NF4_ERR_NULL),
    ("merge null out", lambda L: L.nf4_lora_merge(ctypes.byref(_w()), A, A, 16, 2.0, None, 1, None), nf4.NF4_ERR_NULL),
    ("merge cols%8", lambda L: L.nf4_lora_merge(ctypes.byref(_w(cols=100)), A, A, 16, 2.0, A, 1, None), nf4.NF4_ERR_SIZE),
    ("merge rank 0", lambda L: L.nf4_lora_merge(ctypes.byref(_w()), A, A, 0, 2.0, A, 1, None), nf4.NF4_ERR_SIZE),
    ("merge rank 65", lambda L: L.nf4_lora_merge(ctypes.byref(_w()), A, A, 65, 2.0, A, 1, None), nf4.NF4_ERR_SIZE),
    ("merge scale inf", lambda L: L.nf4_lora_merge(ctypes.byref(_w()), A, A, 16, float("inf"), A, 1, None), nf4.NF4_ERR_SIZE),
    ("merge f32 out", lambda L: L.nf4_lora_merge(ctypes.byref(_w()), A, A, 16, 2.0, A, 0, None), nf4.NF4_ERR_DTYPE),
    ("merge misaligned out", lambda L: L.nf4_lora_merge(ctypes.byref(_w()), A, A, 16, 2.0, A + 2, 2, None), nf4.NF4_ERR_ALIGN),
    ("merge misaligned b", lambda L: L.nf4_lora_merge(ctypes.byref(_w()), A, A + 8, 16, 2.0, A, 1, None), nf4.NF4_ERR_ALIGN),
]


def _batch(L, ws, xs=None, ys=None, count=None, y_dtype=1):
    arr = (nf4.nf4_weight * len(ws))(*ws)
    xs = xs if xs is not None else [A] * len(ws)
    ys = ys if ys is not None else [A2] * len(ws)
    xp = (ctypes.c_void_p * len(xs))(*xs)
    yp = (ctypes.c_void_p * len(ys))(*ys)
    return L.nf4_gemv_batched(arr, len(ws) if count is None else count, xp, yp, y_dtype, None)


def _dqw(**kw):
    return _w(absmax=None, qabsmax=A, absmax2=A2, mean=A2, **kw)


CASES += [
    ("batched null ws", lambda L: L.nf4_gemv_batched(None, 1, (ctypes.c_void_p * 1)(A), (ctypes.c_void_p * 1)(A), 1, None), nf4.NF4_ERR_NULL),
    ("batched count 0", lambda L: _batch(L, [_w()], count=0), nf4.NF4_ERR_SIZE),
    ("batched count 9", lambda L: _batch(L, [_w()] * 9), nf4.NF4_ERR_SIZE),
    ("batched bad dtype", lambda L: _batch(L, [_w()], y_dtype=2), nf4.NF4_ERR_DTYPE),
    ("batched cols%64", lambda L: _batch(L, [_w(), _w(cols=96)]), nf4.NF4_ERR_SIZE),
    ("batched cols>65536", lambda L: _batch(L, [_w(cols=65600)]), nf4.NF4_ERR_SIZE),
    ("batched null x", lambda L: _batch(L, [_w(), _w()], xs=[A, None]), nf4.NF4_ERR_NULL),
    ("batched misaligned y", lambda L: _batch(L, [_w(), _w()], ys=[A2, A2 + 4]), nf4.NF4_ERR_ALIGN),
    ("batched mixed scale forms", lambda L: _batch(L, [_w(), _dqw()]), nf4.NF4_ERR_DTYPE),
    ("batched mixed dq types", lambda L: _batch(L, [_dqw(), _dqw(dq_type=1)]), nf4.NF4_ERR_DTYPE),
    ("batched mixed code books", lambda L: _batch(L, [_w(), _w(quant_type=1)]), nf4.NF4_ERR_DTYPE),
    ("batched bad weight", lambda L: _batch(L, [_w(), _w(blocksize=32)]), nf4.NF4_ERR_BLOCKSIZE),
]


def _dqj(**kw):
    f = dict(absmax=A, nblocks=10, qabsmax=A, absmax2=A2, mean=A2)
    f.update(kw)
    return nf4.nf4_dq_job(**f)


def _dqb(L, jobs, count=None, blocksize2=256, dq_type=0, ws=A, wsb=8 * WS, stream=None):
    arr = (nf4.nf4_dq_job * max(len(jobs), 1))(*jobs)
    return L.nf4_double_quant_batched(arr, len(jobs) if count is None else count, blocksize2, dq_type, ws, wsb, stream)


CASES += [
    ("dq batched null jobs", lambda L: L.nf4_double_quant_batched(None, 1, 256, 0, A, 8 * WS, None), nf4.NF4_ERR_NULL),
    ("dq batched count 0", lambda L: _dqb(L, [_dqj()], count=0), nf4.NF4_ERR_SIZE),
    ("dq batched count 9", lambda L: _dqb(L, [_dqj()] * 9), nf4.NF4_ERR_SIZE),
    ("dq batched blocksize2", lambda L: _dqb(L, [_dqj()], blocksize2=128), nf4.NF4_ERR_BLOCKSIZE),
    ("dq batched dq_type", lambda L: _dqb(L, [_dqj()], dq_type=2), nf4.NF4_ERR_DTYPE),
    ("dq batched workspace small", lambda L: _dqb(L, [_dqj(), _dqj()], wsb=L.nf4_double_quant_batched_workspace(2) - 1), nf4.NF4_ERR_WORKSPACE),
    ("dq batched workspace null", lambda L: _dqb(L, [_dqj()], ws=None), nf4.NF4_ERR_WORKSPACE),
    ("dq batched misaligned workspace", lambda L: _dqb(L, [_dqj()], ws=A + 8), nf4.NF4_ERR_ALIGN),
    ("dq batched null mean", lambda L: _dqb(L, [_dqj(), _dqj(mean=None)]), nf4.NF4_ERR_NULL),
    ("dq batched nblocks 0", lambda L: _dqb(L, [_dqj(), _dqj(nblocks=0)]), nf4.NF4_ERR_SIZE),
    ("dq batched nblocks 2^31", lambda L: _dqb(L, [_dqj(nblocks=1 << 31)]), nf4.NF4_ERR_SIZE),
    ("dq batched misaligned q", lambda L: _dqb(L, [_dqj(), _dqj(qabsmax=A + 1)]), nf4.NF4_ERR_ALIGN),
    ("dq batched misaligned absmax2", lambda L: _dqb(L, [_dqj(absmax2=A2 + 2)]), nf4.NF4_ERR_ALIGN),
]


def _qj(**kw):
    f = dict(x=A, n=128, packed=A, absmax=A2)
    f.update(kw)
    return nf4.nf4_quantize_job(**f)


def _qb(L, jobs, count=None, x_dtype=1, blocksize=64, quant_type=0):
    arr = (nf4.nf4_quantize_job * max(len(jobs), 1))(*jobs)
    return L.nf4_quantize_batched(arr, len(jobs) if count is None else count, x_dtype, blocksize, quant_type, None)


CASES += [
    ("quantize batched null jobs", lambda L: L.nf4_quantize_batched(None, 1, 1, 64, 0, None), nf4.NF4_ERR_NULL),
    ("quantize batched count 0", lambda L: _qb(L, [_qj()], count=0), nf4.NF4_ERR_SIZE),
    ("quantize batched count 9", lambda L: _qb(L, [_qj()] * 9), nf4.NF4_ERR_SIZE),
    ("quantize batched dtype", lambda L: _qb(L, [_qj()], x_dtype=5), nf4.NF4_ERR_DTYPE),
    ("quantize batched blocksize", lambda L: _qb(L, [_qj()], blocksize=128), nf4.NF4_ERR_BLOCKSIZE),
    ("quantize batched quant_type", lambda L: _qb(L, [_qj()], quant_type=2), nf4.NF4_ERR_DTYPE),
    ("quantize batched null packed", lambda L: _qb(L, [_qj(), _qj(packed=None)]), nf4.NF4_ERR_NULL),
    ("quantize batched n 0", lambda L: _qb(L, [_qj(), _qj(n=0)]), nf4.NF4_ERR_SIZE),
    ("quantize batched n 2^40", lambda L: _qb(L, [_qj(n=1 << 40)]), nf4.NF4_ERR_SIZE),
    ("quantize batched misaligned x", lambda L: _qb(L, [_qj(), _qj(x=A + 2)]), nf4.NF4_ERR_ALIGN),
    ("quantize batched misaligned absmax", lambda L: _qb(L, [_qj(absmax=A2 + 2)]), nf4.NF4_ERR_ALIGN),
]


def test_dq_batched_workspace_size(L):
    one = L.nf4_double_quant_workspace(1)
    assert [L.nf4_double_quant_batched_workspace(c) for c in (0, 1, 7, 8, 9)] == [0, one, 7 * one, 8 * one, 0]


@pytest.mark.parametrize("name,call,code", CASES, ids=[c[0] for c in CASES])
def test_invalid_arguments_rejected_on_host(L, name, call, code):
    rc = call(L)
    assert rc == code, (name, rc, nf4.nf4_last_error())
    msg = nf4.nf4_last_error()
    assert msg.startswith("nf4_"), msg


def test_codebook_null(L):
    assert L.nf4_codebook(None) == nf4.NF4_ERR_NULL


def test_fp4_codebook_bit_identical_to_oracle():
    """The library's FP4 code book (host call) equals the oracle's, bit for bit
    (both derived independently from the E2M1 definition)."""
    import numpy as np
    import oracle
    got = np.array(nf4.nf4_codebook_fp4(), dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), oracle.fp4_codebook().view(np.uint32))


# ------------------------------------------------- binding-side weight checks

def _cpu_weight(rows, cols, dq=True, short=None, dtype_swap=None):
    import torch
    n = rows * cols
    nb = -(-n // 64)
    parts = dict(packed=torch.zeros((n + 1) // 2, dtype=torch.uint8))
    if dq:
        parts.update(qabsmax=torch.zeros(nb, dtype=torch.int8), absmax2=torch.zeros(-(-nb // 256), dtype=torch.float32),
                     mean=torch.zeros(1, dtype=torch.float32))
    else:
        parts.update(absmax=torch.zeros(nb, dtype=torch.float32))
    if short:
        parts[short] = parts[short][:-1]
    if dtype_swap:
        name, dt = dtype_swap
        parts[name] = parts[name].to(dt)
    return nf4.NF4Weight(rows=rows, cols=cols, **parts)


@pytest.mark.parametrize("short", ["packed", "qabsmax", "absmax2", "mean"])
def test_weight_descriptor_rejects_short_buffers(short):
    """The C ABI takes bare pointers and cannot see sizes, so the binding
    checks every buffer of a weight against its rows and cols before a call."""
    w = _cpu_weight(300, 128, dq=True, short=short)
    with pytest.raises(ValueError, match=short):
        w.check()


def test_weight_descriptor_rejects_short_plain_absmax_and_wrong_dtypes():
    import torch
    with pytest.raises(ValueError, match="absmax"):
        _cpu_weight(33, 192, dq=False, short="absmax").check()
    with pytest.raises(TypeError, match="absmax2"):
        _cpu_weight(33, 192, dq=True, dtype_swap=("absmax2", torch.float64)).check()
    with pytest.raises(TypeError, match="packed"):
        _cpu_weight(33, 192, dq=True, dtype_swap=("packed", torch.int16)).check()
    with pytest.raises(ValueError, match="required"):
        nf4.NF4Weight(torch.zeros(64, dtype=torch.uint8), 1, 128, qabsmax=torch.zeros(2, dtype=torch.int8)).check()


def test_weight_descriptor_rejects_host_tensors_and_mixed_devices():
    """Buffers of the right sizes on the host are still refused (the library
    takes device pointers only): nothing reaches the C ABI."""
    w = _cpu_weight(64, 64, dq=True)
    with pytest.raises(ValueError, match="device tensors"):
        w.check()
    with pytest.raises(ValueError, match="device tensors"):
        nf4.nf4_gemv(w, __import__("torch").zeros((1, 64), dtype=__import__("torch").bfloat16))


def _build_lut_fn(L):
    out = subprocess.run(["nm", "-D", "--defined-only", nf4.LIB_PATH], capture_output=True, text=True, check=True).stdout
    name = next(ln.split()[-1] for ln in out.splitlines() if "9build_lut" in ln)
    f = getattr(L, name)
    f.restype = ctypes.c_bool
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_char_p, ctypes.c_size_t]
    return f


def test_quantizer_table_self_check_reports_instead_of_aborting(L):
    """The quantizer's bucket table is built and checked on the host at first
    use.  A code book that breaks the table's assumption (two decision
    thresholds inside one bucket) makes the check return false with a reason;
    it no longer ends the caller's process.  The real code books pass."""
    f = _build_lut_fn(L)
    lut = ctypes.create_string_buffer(48 * 8)
    err = ctypes.create_string_buffer(160)

    def codebook_struct(levels):
        levels = np.asarray(levels, dtype=np.float32)
        mids = (levels[:-1].astype(np.float64) + levels[1:]) / 2  # thresholds between neighbours
        thresh = np.concatenate([mids.astype(np.float32), [np.inf]]).astype(np.float32)
        return np.concatenate([levels, thresh]).astype(np.float32)

    good = codebook_struct(oracle.codebook())
    assert f(good.ctypes.data, ctypes.addressof(lut), err, 160)
    assert err.value == b""
    lv = oracle.codebook().copy()
    lv[12], lv[13] = np.float32(0.3), np.float32(0.3001)   # thresholds 0.30005 and ~0.37: same bucket [0.25, 0.3125)
    lv[11] = np.float32(0.26)
    bad = codebook_struct(lv)
    assert not f(bad.ctypes.data, ctypes.addressof(lut), err, 160)
    assert b"two decision thresholds" in err.value
