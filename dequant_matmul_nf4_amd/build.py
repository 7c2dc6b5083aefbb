"""Builds libnf4.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m dequant_matmul_nf4_amd.build [--sanitize]

Every source is compiled with hipcc for gfx950 only, without fused
multiply-add contraction (the quantizer's arithmetic is specified operation by
operation) and without packed-fp32 instructions.

--sanitize builds a second copy, _build/sanitize/libnf4.so, whose host code
(argument checks, code-book derivation, launch planning) is instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer; the device code is the same.
It is for host-only runs: load it with the sanitizer runtime preloaded
(sanitizer_runtime() names it) and NF4_LIBRARY pointing at it.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libnf4.so")
SAN_BUILD = os.path.join(BUILD, "sanitize")
SAN_LIB = os.path.join(SAN_BUILD, "libnf4.so")
# host-side instrumentation only: each option is routed to the host pass
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wno-unused-function",
          f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, src + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip", *DEVICE]
    else:
        cmd[1:1] = ["-D__HIP_PLATFORM_AMD__"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out_dir, lib, extra = (SAN_BUILD, SAN_LIB, SANITIZE) if sanitize else (BUILD, LIB, [])
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, out_dir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources")
    return lib


CALIB = os.path.join(PKG, "calib")
CALIB_LIB = os.path.join(PKG, "libnf4_calib.so")


def build_calib(verbose: bool = False) -> str:
    """The benchmark's calibration kernels (a plain streaming read), built
    into their own library; the NF4 library does not contain them."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CALIB) if f.endswith(".hip"))
    objs = []
    for src in srcs:
        obj = os.path.join(BUILD, "calib_" + src + ".o")
        cmd = [hipcc(), "-x", "hip", *DEVICE, *COMMON, "-c", os.path.join(CALIB, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        objs.append(obj)
    tmp = CALIB_LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, CALIB_LIB)
    if verbose:
        print(f"built {CALIB_LIB}")
    return CALIB_LIB


def sanitizer_runtime() -> str:
    """The compiler's AddressSanitizer runtime (it carries the
    UndefinedBehaviorSanitizer handlers too), to preload into an
    uninstrumented interpreter that loads the sanitized library."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        libdir = subprocess.run([hipcc(), "-print-libgcc-file-name"], capture_output=True, text=True).stdout.strip()
        path = os.path.join(os.path.dirname(libdir), "libclang_rt.asan-x86_64.so")
    if not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime of hipcc's clang was not found")
    return path


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
    if "--sanitize" not in sys.argv[1:]:
        build_calib(verbose=True)
    sys.exit(0)
