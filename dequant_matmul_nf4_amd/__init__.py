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
# NF4_LIBRARY selects another build of the same library (the sanitizer build
# of the host-only tests); by default the in-tree libnf4.so is loaded.
LIB_PATH = os.environ.get("NF4_LIBRARY") or os.path.join(_HERE, "libnf4.so")

(NF4_OK, NF4_ERR_NULL, NF4_ERR_SIZE, NF4_ERR_BLOCKSIZE, NF4_ERR_ALIGN, NF4_ERR_DTYPE, NF4_ERR_WORKSPACE, NF4_ERR_DEVICE,
 NF4_ERR_INTERNAL) = range(9)
NF4_F32, NF4_BF16, NF4_F16 = 0, 1, 2
NF4_DQ_INT8, NF4_DQ_FP8 = 0, 1
NF4_QT_NF4, NF4_QT_FP4 = 0, 1
BLOCKSIZE, BLOCKSIZE2 = 64, 256

EXPORTS = (
    "nf4_last_error", "nf4_codebook", "nf4_codebook_fp4", "nf4_quantize", "nf4_quantize_fp4", "nf4_double_quant_workspace",
    "nf4_double_quant", "nf4_e4m3_ratio", "nf4_double_quant_f8", "nf4_dequantize", "nf4_gemv", "nf4_gemm_workspace", "nf4_gemm", "nf4_gemm_dx_workspace",
    "nf4_gemm_dx", "nf4_lora_grads_workspace", "nf4_lora_grads", "nf4_lora_merge", "nf4_double_quant_noalloc",
    "nf4_gemv_batched", "nf4_double_quant_batched_workspace", "nf4_double_quant_batched", "nf4_quantize_batched",
)


class NF4Error(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


class nf4_quantize_job(ctypes.Structure):
    """Mirror of `struct nf4_quantize_job` in include/nf4.h."""
    _fields_ = [("x", ctypes.c_void_p), ("n", ctypes.c_int64), ("packed", ctypes.c_void_p), ("absmax", ctypes.c_void_p)]


class nf4_dq_job(ctypes.Structure):
    """Mirror of `struct nf4_dq_job` in include/nf4.h."""
    _fields_ = [
        ("absmax", ctypes.c_void_p), ("nblocks", ctypes.c_int64), ("qabsmax", ctypes.c_void_p),
        ("absmax2", ctypes.c_void_p), ("mean", ctypes.c_void_p),
    ]


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
        "nf4_double_quant_noalloc": (ctypes.c_int, [vp, i64, i32, vp, vp, vp, vp]),
        "nf4_quantize_batched": (ctypes.c_int, [ctypes.POINTER(nf4_quantize_job), i32, ctypes.c_int, i32, i32, vp]),
        "nf4_double_quant_batched_workspace": (sz, [i32]),
        "nf4_double_quant_batched": (ctypes.c_int, [ctypes.POINTER(nf4_dq_job), i32, i32, i32, vp, sz, vp]),
        "nf4_e4m3_ratio": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float)]),
        "nf4_dequantize": (ctypes.c_int, [wp, vp, ctypes.c_int, vp]),
        "nf4_gemv": (ctypes.c_int, [wp, vp, i64, vp, ctypes.c_int, vp]),
        "nf4_gemv_batched": (ctypes.c_int, [wp, i32, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int, vp]),
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


def _alloc_on(stream, *shape_dtype_device):
    """torch.empty(shape, dtype, device) for a tensor the library writes on
    `stream`.  When that is not the current stream, the tensor is recorded on
    it, so the caching allocator does not hand its memory to another
    allocation before the work queued on `stream` has finished."""
    torch = _torch()
    shape, dtype, device = shape_dtype_device
    t = torch.empty(shape, dtype=dtype, device=device)
    if stream is not None and stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)
    return t


def _as_rows(t, n: int, stream=None):
    """t as a [-, n] matrix.  A non-contiguous t is copied by reshape; that
    copy is a tensor of the binding's own, read by work queued on `stream`,
    so it is recorded there like the buffers _alloc_on makes (else the
    caching allocator could reuse its memory while the kernel still reads
    it)."""
    torch = _torch()
    t2 = t.reshape(-1, n)
    if (stream is not None and t2.is_cuda and t2.untyped_storage().data_ptr() != t.untyped_storage().data_ptr()
            and stream != torch.cuda.current_stream(t2.device)):
        t2.record_stream(stream)
    return t2


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


def _same_device(dev, *ts):
    for t in ts:
        if t is not None and t.device != dev:
            raise ValueError(f"tensor on {t.device}, expected {dev}")


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

    def check(self) -> None:
        """Host-side check of the buffers against rows and cols: the C ABI
        takes bare pointers, so a buffer shorter than the shape implies would
        be read past its end on the device.  Raises ValueError or TypeError."""
        torch = _torch()
        if int(self.rows) < 1 or int(self.cols) < 1:
            raise ValueError(f"bad shape {self.rows} x {self.cols}")
        n = int(self.rows) * int(self.cols)
        nb = -(-n // BLOCKSIZE)
        need = [("packed", self.packed, (n + 1) // 2, (torch.uint8,))]
        if self.absmax is not None:
            need.append(("absmax", self.absmax, nb, (torch.float32,)))
        else:
            if self.qabsmax is None or self.absmax2 is None or self.mean is None:
                raise ValueError("without absmax, qabsmax, absmax2 and mean are all required")
            need += [("qabsmax", self.qabsmax, nb, (torch.int8, torch.uint8)),
                     ("absmax2", self.absmax2, -(-nb // BLOCKSIZE2), (torch.float32,)),
                     ("mean", self.mean, 1, (torch.float32,))]
        dev = None
        for name, t, count, dtypes in need:
            if t.dtype not in dtypes:
                raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
            if t.numel() < count:
                raise ValueError(f"{name} holds {t.numel()} elements; a {self.rows} x {self.cols} weight needs {count}")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{name} is on {t.device}, the packed codes on {dev}")
        if dev is None or dev.type != "cuda":
            raise ValueError("the weight's buffers must be device tensors")

    @property
    def device(self):
        return self.packed.device

    def c_struct(self) -> nf4_weight:
        self.check()
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
        packed = _alloc_on(stream, ((n + 1) // 2,), torch.uint8, x.device)
    if absmax is None:
        absmax = _alloc_on(stream, ((n + 63) // 64,), torch.float32, x.device)
    _need_cuda(packed, absmax)
    _same_device(x.device, packed, absmax)
    if packed.dtype != torch.uint8 or absmax.dtype != torch.float32:
        raise TypeError("packed must be uint8 and absmax float32")
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
        qabsmax = _alloc_on(stream, (nb,), torch.uint8 if fp8 else torch.int8, dev)
    absmax2 = _alloc_on(stream, ((nb + 255) // 256,), torch.float32, dev) if absmax2 is None else absmax2
    mean = _alloc_on(stream, (1,), torch.float32, dev) if mean is None else mean
    wsb = nf4_double_quant_workspace(nb)
    if workspace is None:
        workspace = _alloc_on(stream, (wsb,), torch.uint8, dev)
    _need_cuda(qabsmax, absmax2, mean, workspace)
    _same_device(dev, qabsmax, absmax2, mean, workspace)
    if absmax2.dtype != torch.float32 or mean.dtype != torch.float32 or qabsmax.element_size() != 1:
        raise TypeError("qabsmax must hold bytes, absmax2 and mean float32")
    if qabsmax.numel() < nb or absmax2.numel() < (nb + 255) // 256 or mean.numel() < 1:
        raise ValueError("output buffers too small")
    fn = lib().nf4_double_quant_f8 if fp8 else lib().nf4_double_quant
    _check(fn(_ptr(absmax), nb, BLOCKSIZE2, _ptr(qabsmax), _ptr(absmax2), _ptr(mean),
              _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return qabsmax, absmax2, mean


def nf4_quantize_batched(xs, outs=None, stream=None, fp4=False):
    """nf4_quantize (fp4=True: nf4_quantize_fp4) of 1 to 8 tensors of one dtype
    in one launch; each tensor's outputs are those of the single call.
    outs: optional list of (packed, absmax) per tensor.  Returns the list of
    (packed, absmax)."""
    torch = _torch()
    xs = list(xs)
    if not 1 <= len(xs) <= 8:
        raise ValueError("1 to 8 tensors")
    _need_cuda(*xs)
    dt = xs[0].dtype
    if dt not in (torch.float32, torch.bfloat16) or any(x.dtype != dt for x in xs):
        raise TypeError("all tensors float32, or all bf16")
    for x in xs:
        if not x.is_contiguous():
            raise ValueError("tensors must be contiguous")
    dev = xs[0].device
    if outs is None:
        outs = [(_alloc_on(stream, ((x.numel() + 1) // 2,), torch.uint8, dev),
                 _alloc_on(stream, ((x.numel() + 63) // 64,), torch.float32, dev)) for x in xs]
    outs = [tuple(o) for o in outs]
    if len(outs) != len(xs):
        raise ValueError("one (packed, absmax) per tensor")
    for x, (p, a) in zip(xs, outs):
        _need_cuda(p, a)
        _same_device(dev, x, p, a)
        if p.dtype != torch.uint8 or a.dtype != torch.float32:
            raise TypeError("packed must be uint8 and absmax float32")
        if p.numel() < (x.numel() + 1) // 2 or a.numel() < (x.numel() + 63) // 64:
            raise ValueError("output buffers too small")
    jobs = (nf4_quantize_job * len(xs))(*[nf4_quantize_job(_ptr(x), x.numel(), _ptr(p), _ptr(a))
                                          for x, (p, a) in zip(xs, outs)])
    _check(lib().nf4_quantize_batched(jobs, len(xs), NF4_BF16 if dt == torch.bfloat16 else NF4_F32, BLOCKSIZE,
                                      NF4_QT_FP4 if fp4 else NF4_QT_NF4, _stream(stream)))
    return outs


def nf4_double_quant_batched(absmaxes, outs=None, workspace=None, stream=None, fp8=False):
    """nf4_double_quant (fp8=True: nf4_double_quant_f8) of 1 to 8 scale arrays
    in one pair of launches; each array's outputs are those of the single
    call.  outs: optional list of (qabsmax, absmax2, mean) per array.
    Returns the list of (qabsmax, absmax2, mean)."""
    torch = _torch()
    absmaxes = list(absmaxes)
    if not 1 <= len(absmaxes) <= 8:
        raise ValueError("1 to 8 scale arrays")
    _need_cuda(*absmaxes)
    dev = absmaxes[0].device
    if outs is None:
        outs = [(_alloc_on(stream, (a.numel(),), torch.uint8 if fp8 else torch.int8, dev),
                 _alloc_on(stream, ((a.numel() + 255) // 256,), torch.float32, dev),
                 _alloc_on(stream, (1,), torch.float32, dev)) for a in absmaxes]
    outs = [tuple(o) for o in outs]
    if len(outs) != len(absmaxes):
        raise ValueError("one (qabsmax, absmax2, mean) per array")
    for a, (q, s2, mu) in zip(absmaxes, outs):
        if a.dtype != torch.float32:
            raise TypeError("absmax must be float32")
        _need_cuda(q, s2, mu)
        _same_device(dev, a, q, s2, mu)
        if s2.dtype != torch.float32 or mu.dtype != torch.float32 or q.element_size() != 1:
            raise TypeError("qabsmax must hold bytes, absmax2 and mean float32")
        if q.numel() < a.numel() or s2.numel() < (a.numel() + 255) // 256 or mu.numel() < 1:
            raise ValueError("output buffers too small")
    wsb = lib().nf4_double_quant_batched_workspace(len(absmaxes))
    if workspace is None:
        workspace = _alloc_on(stream, (wsb,), torch.uint8, dev)
    _need_cuda(workspace)
    _same_device(dev, workspace)
    jobs = (nf4_dq_job * len(absmaxes))(*[nf4_dq_job(_ptr(a), a.numel(), _ptr(q), _ptr(s2), _ptr(mu))
                                          for a, (q, s2, mu) in zip(absmaxes, outs)])
    _check(lib().nf4_double_quant_batched(jobs, len(absmaxes), BLOCKSIZE2, NF4_DQ_FP8 if fp8 else NF4_DQ_INT8,
                                          _ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _stream(stream)))
    return outs


def nf4_double_quant_noalloc(absmax, qabsmax, absmax2, mean, stream=None):
    """nf4_double_quant (int8 second level) through the entry point that
    allocates nothing: the outputs are the caller's and the partial sums use
    the library's static device scratch.  Returns (qabsmax, absmax2, mean)."""
    torch = _torch()
    _need_cuda(absmax, qabsmax, absmax2, mean)
    _same_device(absmax.device, qabsmax, absmax2, mean)
    if absmax.dtype != torch.float32 or absmax2.dtype != torch.float32 or mean.dtype != torch.float32:
        raise TypeError("absmax, absmax2 and mean must be float32")
    if qabsmax.dtype != torch.int8:
        raise TypeError("qabsmax must be int8")
    nb = absmax.numel()
    if qabsmax.numel() < nb or absmax2.numel() < (nb + 255) // 256 or mean.numel() < 1:
        raise ValueError("output buffers too small")
    _check(lib().nf4_double_quant_noalloc(_ptr(absmax), nb, BLOCKSIZE2, _ptr(qabsmax), _ptr(absmax2), _ptr(mean),
                                          _stream(stream)))
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


def quantize_weights(ws, double_quant: bool = True, stream=None, dq_type: str = "int8",
                     quant_type: str = "nf4") -> list:
    """quantize_weight for 1 to 8 2-D weights of one dtype (for instance the
    seven weights of a transformer layer) through one nf4_quantize_batched
    launch and one nf4_double_quant_batched call; each NF4Weight holds
    exactly what quantize_weight gives for that weight."""
    if quant_type not in ("nf4", "fp4"):
        raise ValueError("quant_type must be 'nf4' or 'fp4'")
    if dq_type not in ("int8", "fp8"):
        raise ValueError("dq_type must be 'int8' or 'fp8'")
    ws = list(ws)
    if any(w.dim() != 2 for w in ws):
        raise ValueError("weights must be 2-D")
    qt = NF4_QT_FP4 if quant_type == "fp4" else NF4_QT_NF4
    codes = nf4_quantize_batched(ws, stream=stream, fp4=qt == NF4_QT_FP4)
    if not double_quant:
        return [NF4Weight(p, w.shape[0], w.shape[1], absmax=a, quant_type=qt) for w, (p, a) in zip(ws, codes)]
    fp8 = dq_type == "fp8"
    scales = nf4_double_quant_batched([a for _, a in codes], stream=stream, fp8=fp8)
    return [NF4Weight(p, w.shape[0], w.shape[1], qabsmax=q, absmax2=s2, mean=mu,
                      dq_type=NF4_DQ_FP8 if fp8 else NF4_DQ_INT8, quant_type=qt)
            for w, (p, _), (q, s2, mu) in zip(ws, codes, scales)]


def nf4_dequantize(w: NF4Weight, out=None, out_dtype=None, stream=None):
    torch = _torch()
    cs = w.c_struct()
    if out is None:
        out = _alloc_on(stream, (w.rows, w.cols), out_dtype or torch.bfloat16, w.device)
    _need_cuda(out)
    _same_device(w.device, out)
    if out.numel() != w.rows * w.cols:
        raise ValueError("out has the wrong size")
    _check(lib().nf4_dequantize(ctypes.byref(cs), _ptr(out), _dtype_code(out), _stream(stream)))
    return out


def nf4_gemv(w: NF4Weight, x, y=None, y_dtype=None, stream=None):
    """y = x . deq(W)^T for x bf16 [m, cols] with 1 <= m <= 16."""
    torch = _torch()
    x2 = _as_rows(x, w.cols, stream)
    _need_cuda(x2)
    if x2.dtype != torch.bfloat16:
        raise TypeError("x must be bf16")
    m = x2.shape[0]
    cs = w.c_struct()
    if y is None:
        y = _alloc_on(stream, (m, w.rows), y_dtype or torch.bfloat16, x.device)
    _need_cuda(y)
    _same_device(w.device, x2, y)
    if y.numel() != m * w.rows:
        raise ValueError("y has the wrong size")
    _check(lib().nf4_gemv(ctypes.byref(cs), _ptr(x2), m, _ptr(y), _dtype_code(y), _stream(stream)))
    return y


def nf4_gemv_batched(ws, xs, ys=None, y_dtype=None, stream=None):
    """ys[i] = xs[i] . deq(ws[i])^T at m = 1 for several weights in one launch;
    xs[i] is bf16 [1, cols_i] (the same tensor may serve several weights).
    Returns the list of outputs."""
    torch = _torch()
    ws, xs = list(ws), list(xs)
    if len(ws) != len(xs) or not 1 <= len(ws) <= 8:
        raise ValueError("ws and xs must be lists of the same length, 1 to 8")
    structs = (nf4_weight * len(ws))(*[w.c_struct() for w in ws])
    if ys is None:
        ys = [_alloc_on(stream, (1, w.rows), y_dtype or torch.bfloat16, xs[i].device) for i, w in enumerate(ws)]
    ys = list(ys)
    for w, x, y in zip(ws, xs, ys):
        _need_cuda(x, y)
        _same_device(w.device, x, y)
        if x.dtype != torch.bfloat16 or x.numel() != w.cols:
            raise ValueError("each x must be bf16 with cols values (m = 1)")
        if y.numel() != w.rows or y.dtype != ys[0].dtype:
            raise ValueError("each y must hold rows values, all of one dtype")
    xp = (ctypes.c_void_p * len(ws))(*[_ptr(x) for x in xs])
    yp = (ctypes.c_void_p * len(ws))(*[_ptr(y) for y in ys])
    _check(lib().nf4_gemv_batched(structs, len(ws), xp, yp, _dtype_code(ys[0]), _stream(stream)))
    return ys


def nf4_gemm(w: NF4Weight, x, y=None, lora_a=None, lora_b=None, lora_scale: float = 0.0,
             workspace=None, stream=None):
    """y = x . deq(W)^T + lora_scale . (x . A^T) . B^T, bf16 in and out."""
    torch = _torch()
    x2 = _as_rows(x, w.cols, stream)
    _need_cuda(x2, lora_a, lora_b)
    m = x2.shape[0]
    r = 0 if lora_a is None else lora_a.shape[0]
    cs = w.c_struct()
    if y is None:
        y = _alloc_on(stream, (m, w.rows), torch.bfloat16, x.device)
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
        workspace = _alloc_on(stream, (wsb,), torch.uint8, x.device)
    _need_cuda(workspace)
    _same_device(w.device, x2, y, lora_a, lora_b, workspace)
    wsn = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().nf4_gemm(ctypes.byref(cs), _ptr(x2), m, _ptr(y), _ptr(lora_a), _ptr(lora_b), r,
                          float(lora_scale), _ptr(workspace), wsn, _stream(stream)))
    return y


def nf4_gemm_dx(w: NF4Weight, dy, dx=None, lora_a=None, lora_b=None, lora_scale: float = 0.0,
                workspace=None, stream=None):
    """dx = dy . deq(W) + lora_scale . (dy . B) . A, bf16 in and out."""
    torch = _torch()
    dy2 = _as_rows(dy, w.rows, stream)
    _need_cuda(dy2, lora_a, lora_b)
    m = dy2.shape[0]
    r = 0 if lora_a is None else lora_a.shape[0]
    cs = w.c_struct()
    if dx is None:
        dx = _alloc_on(stream, (m, w.cols), torch.bfloat16, dy.device)
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
        workspace = _alloc_on(stream, (wsb,), torch.uint8, dy.device)
    _need_cuda(workspace)
    _same_device(w.device, dy2, dx, lora_a, lora_b, workspace)
    wsn = 0 if workspace is None else workspace.numel() * workspace.element_size()
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
    x2 = _as_rows(x, cols, stream)
    dy2 = _as_rows(dy, rows, stream)
    _need_cuda(x2, dy2, lora_a, lora_b)
    m = x2.shape[0]
    if dy2.shape[0] != m or tuple(lora_b.shape) != (rows, r):
        raise ValueError("shapes must be x [m, cols], dy [m, rows], A [r, cols], B [rows, r]")
    for t in (x2, dy2, lora_a, lora_b):
        if t.dtype != torch.bfloat16:
            raise TypeError("x, dy, lora_a and lora_b must be bf16")
    if da is None and "da" in want:
        da = _alloc_on(stream, (r, cols), torch.float32, x.device)
    if db is None and "db" in want:
        db = _alloc_on(stream, (rows, r), torch.float32, x.device)
    for t, shape in ((da, (r, cols)), (db, (rows, r))):
        if t is not None:
            _need_cuda(t)
            if t.dtype != torch.float32 or t.numel() != shape[0] * shape[1]:
                raise ValueError("da and db must be float32 [r, cols] and [rows, r]")
    wsb = nf4_lora_grads_workspace(m, rows, cols, r)
    if workspace is None:
        workspace = _alloc_on(stream, (max(wsb, 1),), torch.uint8, x.device)
    _need_cuda(workspace)
    _same_device(x.device, dy2, lora_a, lora_b, da, db, workspace)
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
    cs = w.c_struct()
    if out is None:
        out = _alloc_on(stream, (w.rows, w.cols), out_dtype or torch.bfloat16, lora_a.device)
    _need_cuda(out)
    _same_device(w.device, lora_a, lora_b, out)
    if out.numel() != w.rows * w.cols:
        raise ValueError("out has the wrong size")
    _check(lib().nf4_lora_merge(ctypes.byref(cs), _ptr(lora_a), _ptr(lora_b), r, float(lora_scale), _ptr(out),
                                _dtype_code(out), _stream(stream)))
    return out
