"""Python binding of libnf4.so, the NF4 weight library for MI355X (gfx950).

Argument marshalling only: every function below checks shapes and dtypes of
torch tensors, passes their device pointers and the current HIP stream to the
C entry point of the same name (declared in include/nf4.h) and raises
NF4Error on a non-zero status.  All arithmetic runs in the library's HIP
kernels; there is no fallback.  torch supplies device memory and streams.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnf4.so")

NF4_OK, NF4_ERR_NULL, NF4_ERR_SIZE, NF4_ERR_BLOCKSIZE, NF4_ERR_ALIGN, NF4_ERR_DTYPE, NF4_ERR_WORKSPACE, NF4_ERR_DEVICE = range(8)
NF4_F32, NF4_BF16, NF4_F16 = 0, 1, 2
NF4_DQ_INT8, NF4_DQ_FP8 = 0, 1
NF4_QT_NF4, NF4_QT_FP4 = 0, 1
BLOCKSIZE, BLOCKSIZE2 = 64, 256

EXPORTS = (
    "nf4_last_error", "nf4_codebook", "nf4_codebook_fp4", "nf4_quantize", "nf4_quantize_fp4", "nf4_double_quant_workspace",
    "nf4_double_quant", "nf4_e4m3_ratio", "nf4_double_quant_f8", "nf4_dequantize", "nf4_gemv", "nf4_gemm_workspace", "nf4_gemm", "nf4_gemm_dx_workspace",
    "nf4_gemm_dx", "nf4_lora_grads_workspace", "nf4_lora_grads", "nf4_lora_merge",
)


class NF4Error(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


class nf4_weight(ctypes.Structure):
    """Mirror of `struct nf4_weight` in include/nf4.h."""
    _fields_ = [
        ("packed", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
        ("blocksize", ctypes.c_int32), ("absmax", ctypes.c_void_p), ("qabsmax", ctypes.c_void_p),
        ("absmax2", ctypes.c_void_p), ("mean", ctypes.c_void_p), ("blocksize2", ctypes.c_int32),
        ("dq_type", ctypes.c_int32), ("quant_type", ctypes.c_int32),
    ]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m dequant_matmul_nf4_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    wp = ctypes.POINTER(nf4_weight)
    sig = {
        "nf4_last_error": (ctypes.c_char_p, []),
        "nf4_codebook": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float)]),
        "nf4_codebook_fp4": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float)]),
        "nf4_quantize": (ctypes.c_int, [vp, ctypes.c_int, i64, i32, vp, vp, vp]),
        "nf4_quantize_fp4": (ctypes.c_int, [vp, ctypes.c_int, i64, i32, vp, vp, vp]),
        "nf4_double_quant_workspace": (sz, [i64]),
        "nf4_double_quant": (ctypes.c_int, [vp, i64, i32, vp, vp, vp, vp, sz, vp]),
        "nf4_double_quant_f8": (ctypes.c_int, [vp, i64, i32, vp, vp, vp, vp, sz, vp]),
        "nf4_e4m3_ratio": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float)]),
        "nf4_dequantize": (ctypes.c_int, [wp, vp, ctypes.c_int, vp]),
        "nf4_gemv": (ctypes.c_int, [wp, vp, i64, vp, ctypes.c_int, vp]),
        "nf4_gemm_workspace": (sz, [i64, i64, i32]),
        "nf4_gemm": (ctypes.c_int, [wp, vp, i64, vp, vp, vp, i32, ctypes.c_float, vp, sz, vp]),
        "nf4_gemm_dx_workspace": (sz, [i64, i64, i32]),
        "nf4_gemm_dx": (ctypes.c_int, [wp, vp, i64, vp, vp, vp, i32, ctypes.c_float, vp, sz, vp]),
        "nf4_lora_grads_workspace": (sz, [i64, i64, i64, i32]),
        "nf4_lora_grads": (ctypes.c_int, [vp, vp, i64, i64, i64, vp, vp, i32, ctypes.c_float, vp, vp, vp, sz, vp]),
        "nf4_lora_merge": (ctypes.c_int, [wp, vp, vp, i32, ctypes.c_float, vp, ctypes.c_int, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != NF4_OK:
        raise NF4Error(rc, lib().nf4_last_error().decode())


def nf4_last_error() -> str:
    return lib().nf4_last_error().decode()


def nf4_codebook():
    """The 16 NF4 levels (host call, needs no GPU) as a list of floats."""
    out = (ctypes.c_float * 16)()
    _check(lib().nf4_codebook(out))
    return list(out)


def nf4_codebook_fp4():
    """The 16 FP4 levels by code (E2M1 value / 6; host call, needs no GPU)."""
    out = (ctypes.c_float * 16)()
    _check(lib().nf4_codebook_fp4(out))
    return list(out)


def nf4_e4m3_ratio():
    """fl32(e4m3(q) / 448) for the 256 float8 codes (host call, needs no GPU)."""
    out = (ctypes.c_float * 256)()
    _check(lib().nf4_e4m3_ratio(out))
    return list(out)


def nf4_double_quant_workspace(nblocks: int) -> int:
    return int(lib().nf4_double_quant_workspace(nblocks))


def nf4_gemm_workspace(m: int, rows: int, r: int) -> int:
    return int(lib().nf4_gemm_workspace(m, rows, r))


def nf4_gemm_dx_workspace(m: int, rows: int, r: int) -> int:
    return int(lib().nf4_gemm_dx_workspace(m, rows, r))


def nf4_lora_grads_workspace(m: int, rows: int, cols: int, r: int) -> int:
    return int(lib().nf4_lora_grads_workspace(m, rows, cols, r))


# ------------------------------------------------------------- torch glue

def _torch():
    import torch
    return torch


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return NF4_F32
    if t.dtype == torch.bfloat16:
        return NF4_BF16
    if t.dtype == torch.float16:
        return NF4_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


@dataclass
class NF4Weight:
    """A quantized weight W[rows][cols]: packed codes plus one scale form."""
    packed: "object"
    rows: int
    cols: int
    absmax: "object" = None
    qabsmax: "object" = None
    absmax2: "object" = None
    mean: "object" = None
    dq_type: int = 0  # NF4_DQ_INT8 or NF4_DQ_FP8 (second-level codes)
    quant_type: int = 0  # NF4_QT_NF4 or NF4_QT_FP4 (code book of the packed codes)

    @property
    def double_quant(self) -> bool:
        return self.absmax is None

    def c_struct(self) -> nf4_weight:
        return nf4_weight(
            packed=_ptr(self.packed), rows=self.rows, cols=self.cols, blocksize=BLOCKSIZE,
            absmax=_ptr(self.absmax), qabsmax=_ptr(self.qabsmax), absmax2=_ptr(self.absmax2),
            mean=_ptr(self.mean), blocksize2=BLOCKSIZE2, dq_type=self.dq_type, quant_type=self.quant_type,
        )


def nf4_quantize(x, packed=None, absmax=None, stream=None, fp4=False):
    """Blockwise NF4 quantization of all elements of x (float32 or bf16);
    fp4=True: the same steps with the FP4 code book."""
    torch = _torch()
    _need_cuda(x)
    n = x.numel()
    if packed is None:
        packed = torch.empty((n + 1) // 2, dtype=torch.uint8, device=x.device)
    if absmax is None:
        absmax = torch.empty((n + 63) // 64, dtype=torch.float32, device=x.device)
    _need_cuda(packed, absmax)
    if packed.numel() < (n + 1) // 2 or absmax.numel() < (n + 63) // 64:
        raise ValueError("output buffers too small")
    fn = lib().nf4_quantize_fp4 if fp4 else lib().nf4_quantize
    _check(fn(_ptr(x), _dtype_code(x), n, BLOCKSIZE, _ptr(packed), _ptr(absmax), _stream(stream)))
    return packed, absmax


def nf4_double_quant(absmax, qabsmax=None, absmax2=None, mean=None, workspace=None, stream=None, fp8=False):
    """Double quantization of the fp32 scales: returns (qabsmax, absmax2, mean).
    fp8=True: the float8 (E4M3) second level, codes as uint8."""
    torch = _torch()
    _need_cuda(absmax)
    if absmax.dtype != torch.float32:
        raise TypeError("absmax must be float32")
    nb = absmax.numel()
    dev = absmax.device
    if qabsmax is None:
        qabsmax = torch.empty(nb, dtype=torch.uint8 if fp8 else torch.int8, device=dev)
    absmax2 = torch.empty((nb + 255) // 256, dtype=torch.float32, device=dev) if absmax2 is None else absmax2
    mean = torch.empty(1, dtype=torch.float32, device=dev) if mean is None else mean
    wsb = nf4_double_quant_workspace(nb)
    if workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    _need_cuda(qabsmax, absmax2, mean, workspace)
    if qabsmax.numel() < nb or absmax2.numel() < (nb + 255) // 256 or mean.numel() < 1:
        raise ValueError("output buffers too small")
    fn = lib().nf4_double_quant_f8 if fp8 else lib().nf4_double_quant
    _check(fn(_ptr(absmax), nb, BLOCKSIZE2, _ptr(qabsmax), _ptr(absmax2), _ptr(mean),
              _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return qabsmax, absmax2, mean


def quantize_weight(w, double_quant: bool = True, stream=None, dq_type: str = "int8",
                    quant_type: str = "nf4") -> NF4Weight:
    """nf4_quantize (+ nf4_double_quant, int8 or fp8 second level) of a 2-D
    weight into an NF4Weight; quant_type "fp4" uses the FP4 code book."""
    if quant_type not in ("nf4", "fp4"):
        raise ValueError("quant_type must be 'nf4' or 'fp4'")
    qt = NF4_QT_FP4 if quant_type == "fp4" else NF4_QT_NF4
    rows, cols = w.shape
    packed, absmax = nf4_quantize(w, stream=stream, fp4=qt == NF4_QT_FP4)
    if not double_quant:
        return NF4Weight(packed, rows, cols, absmax=absmax, quant_type=qt)
    if dq_type not in ("int8", "fp8"):
        raise ValueError("dq_type must be 'int8' or 'fp8'")
    fp8 = dq_type == "fp8"
    q, s2, mean = nf4_double_quant(absmax, stream=stream, fp8=fp8)
    return NF4Weight(packed, rows, cols, qabsmax=q, absmax2=s2, mean=mean, dq_type=NF4_DQ_FP8 if fp8 else NF4_DQ_INT8,
                     quant_type=qt)


def nf4_dequantize(w: NF4Weight, out=None, out_dtype=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty((w.rows, w.cols), dtype=out_dtype or torch.bfloat16, device=w.packed.device)
    _need_cuda(out)
    if out.numel() != w.rows * w.cols:
        raise ValueError("out has the wrong size")
    cs = w.c_struct()
    _check(lib().nf4_dequantize(ctypes.byref(cs), _ptr(out), _dtype_code(out), _stream(stream)))
    return out


def nf4_gemv(w: NF4Weight, x, y=None, y_dtype=None, stream=None):
    """y = x . deq(W)^T for x bf16 [m, cols] with 1 <= m <= 16."""
    torch = _torch()
    x2 = x.reshape(-1, w.cols)
    _need_cuda(x2)
    if x2.dtype != torch.bfloat16:
        raise TypeError("x must be bf16")
    m = x2.shape[0]
    if y is None:
        y = torch.empty((m, w.rows), dtype=y_dtype or torch.bfloat16, device=x.device)
    _need_cuda(y)
    if y.numel() != m * w.rows:
        raise ValueError("y has the wrong size")
    cs = w.c_struct()
    _check(lib().nf4_gemv(ctypes.byref(cs), _ptr(x2), m, _ptr(y), _dtype_code(y), _stream(stream)))
    return y


def nf4_gemm(w: NF4Weight, x, y=None, lora_a=None, lora_b=None, lora_scale: float = 0.0,
             workspace=None, stream=None):
    """y = x . deq(W)^T + lora_scale . (x . A^T) . B^T, bf16 in and out."""
    torch = _torch()
    x2 = x.reshape(-1, w.cols)
    _need_cuda(x2, lora_a, lora_b)
    m = x2.shape[0]
    r = 0 if lora_a is None else lora_a.shape[0]
    if y is None:
        y = torch.empty((m, w.rows), dtype=torch.bfloat16, device=x.device)
    _need_cuda(y)
    for t in (x2, y, lora_a, lora_b):
        if t is not None and t.dtype != torch.bfloat16:
            raise TypeError("x, y, lora_a and lora_b must be bf16")
    if y.numel() != m * w.rows:
        raise ValueError("y has the wrong size")
    if lora_a is not None and (tuple(lora_a.shape) != (r, w.cols) or lora_b is None or tuple(lora_b.shape) != (w.rows, r)):
        raise ValueError("LoRA shapes must be A [r, cols] and B [rows, r]")
    wsb = nf4_gemm_workspace(m, w.rows, r)
    if wsb and workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=x.device)
    wsn = 0 if workspace is None else workspace.numel() * workspace.element_size()
    cs = w.c_struct()
    _check(lib().nf4_gemm(ctypes.byref(cs), _ptr(x2), m, _ptr(y), _ptr(lora_a), _ptr(lora_b), r,
                          float(lora_scale), _ptr(workspace), wsn, _stream(stream)))
    return y


def nf4_gemm_dx(w: NF4Weight, dy, dx=None, lora_a=None, lora_b=None, lora_scale: float = 0.0,
                workspace=None, stream=None):
    """dx = dy . deq(W) + lora_scale . (dy . B) . A, bf16 in and out."""
    torch = _torch()
    dy2 = dy.reshape(-1, w.rows)
    _need_cuda(dy2, lora_a, lora_b)
    m = dy2.shape[0]
    r = 0 if lora_a is None else lora_a.shape[0]
    if dx is None:
        dx = torch.empty((m, w.cols), dtype=torch.bfloat16, device=dy.device)
    _need_cuda(dx)
    for t in (dy2, dx, lora_a, lora_b):
        if t is not None and t.dtype != torch.bfloat16:
            raise TypeError("dy, dx, lora_a and lora_b must be bf16")
    if dx.numel() != m * w.cols:
        raise ValueError("dx has the wrong size")
    if lora_a is not None and (tuple(lora_a.shape) != (r, w.cols) or lora_b is None or tuple(lora_b.shape) != (w.rows, r)):
        raise ValueError("LoRA shapes must be A [r, cols] and B [rows, r]")
    wsb = nf4_gemm_dx_workspace(m, w.rows, r)
    if wsb and workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dy.device)
    wsn = 0 if workspace is None else workspace.numel() * workspace.element_size()
    cs = w.c_struct()
    _check(lib().nf4_gemm_dx(ctypes.byref(cs), _ptr(dy2), m, _ptr(dx), _ptr(lora_a), _ptr(lora_b), r,
                             float(lora_scale), _ptr(workspace), wsn, _stream(stream)))
    return dx


def nf4_lora_grads(x, dy, lora_a, lora_b, lora_scale: float, da=None, db=None, want=("da", "db"),
                   workspace=None, stream=None):
    """(dA, dB) of the adapters: dA = s (dy B)^T x [r, cols], dB = s dy^T (x A^T)
    [rows, r], float32; a gradient not in `want` (and not given) is None."""
    torch = _torch()
    r, cols = lora_a.shape
    rows = lora_b.shape[0]
    x2 = x.reshape(-1, cols)
    dy2 = dy.reshape(-1, rows)
    _need_cuda(x2, dy2, lora_a, lora_b)
    m = x2.shape[0]
    if dy2.shape[0] != m or tuple(lora_b.shape) != (rows, r):
        raise ValueError("shapes must be x [m, cols], dy [m, rows], A [r, cols], B [rows, r]")
    for t in (x2, dy2, lora_a, lora_b):
        if t.dtype != torch.bfloat16:
            raise TypeError("x, dy, lora_a and lora_b must be bf16")
    if da is None and "da" in want:
        da = torch.empty((r, cols), dtype=torch.float32, device=x.device)
    if db is None and "db" in want:
        db = torch.empty((rows, r), dtype=torch.float32, device=x.device)
    for t, shape in ((da, (r, cols)), (db, (rows, r))):
        if t is not None:
            _need_cuda(t)
            if t.dtype != torch.float32 or t.numel() != shape[0] * shape[1]:
                raise ValueError("da and db must be float32 [r, cols] and [rows, r]")
    wsb = nf4_lora_grads_workspace(m, rows, cols, r)
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=x.device)
    wsn = workspace.numel() * workspace.element_size()
    _check(lib().nf4_lora_grads(_ptr(x2), _ptr(dy2), m, rows, cols, _ptr(lora_a), _ptr(lora_b), r,
                                float(lora_scale), _ptr(da), _ptr(db), _ptr(workspace), wsn, _stream(stream)))
    return da, db


def nf4_lora_merge(w: NF4Weight, lora_a, lora_b, lora_scale: float, out=None, out_dtype=None, stream=None):
    """W' = round(deq(W) + lora_scale . B . A) as a dense [rows, cols] bf16 or fp16 tensor."""
    torch = _torch()
    _need_cuda(lora_a, lora_b)
    r = lora_a.shape[0]
    if lora_a.dtype != torch.bfloat16 or lora_b.dtype != torch.bfloat16:
        raise TypeError("lora_a and lora_b must be bf16")
    if tuple(lora_a.shape) != (r, w.cols) or tuple(lora_b.shape) != (w.rows, r):
        raise ValueError("LoRA shapes must be A [r, cols] and B [rows, r]")
    if out is None:
        out = torch.empty((w.rows, w.cols), dtype=out_dtype or torch.bfloat16, device=lora_a.device)
    _need_cuda(out)
    if out.numel() != w.rows * w.cols:
        raise ValueError("out has the wrong size")
    cs = w.c_struct()
    _check(lib().nf4_lora_merge(ctypes.byref(cs), _ptr(lora_a), _ptr(lora_b), r, float(lora_scale), _ptr(out),
                                _dtype_code(out), _stream(stream)))
    return out
