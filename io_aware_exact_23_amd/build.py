"""Build libfa.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: python -m io_aware_exact_23_amd.build      (or call build()).
Every call recompiles. The library lands next to this file as libfa.so.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")

SOURCES = ["fa_prefill_bf16.hip", "fa_prefill_pp.hip", "fa_prefill_f32.hip", "fa_decode.hip", "fa_standard.hip",
           "fa_backward.hip", "fa_quant_fp8.hip", "fa_prefill_fp8.hip", "fa_api.cpp"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU instructions.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


HOST_SANITIZED_LIB = os.path.join(OUT_DIR, "libfa_hostsan.so")
# AddressSanitizer and UndefinedBehaviorSanitizer on the host code of the C ABI only (argument
# checks, dispatch); each -fsanitize= is preceded by -Xarch_host so no GPU code is built with it.
_HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The compiler's shared AddressSanitizer runtime (it carries the UBSan handlers too); a Python
    process preloads it to load the sanitized library."""
    import glob
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(_hipcc()))), "llvm")
    for root in (llvm, "/opt/rocm/llvm"):
        hits = sorted(glob.glob(os.path.join(root, "lib", "clang", "*", "lib", "linux",
                                             "libclang_rt.asan-x86_64.so")))
        if hits:
            return hits[-1]
    raise RuntimeError("libclang_rt.asan-x86_64.so not found")


def build_host_sanitized() -> str:
    """libfa with fa_api.cpp (the host side of the C ABI) built under ASan and UBSan, linked with
    the ordinary kernel objects (built first if missing). For tests of the argument checks on the
    CPU; it is never the product library."""
    os.makedirs(OUT_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        if src == "fa_api.cpp":
            continue
        obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj if os.path.exists(obj) else _compile(src))
    san_obj = os.path.join(OUT_DIR, "fa_api_hostsan.o")
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g"] + _HOST_SAN
    cmd = [_hipcc(), *flags, "-c", os.path.join(CSRC, "fa_api.cpp"), "-o", san_obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for the sanitized fa_api.cpp:\n{' '.join(cmd)}\n{res.stderr}")
    tmp = HOST_SANITIZED_LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *_HOST_SAN, "-o", tmp, san_obj, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, HOST_SANITIZED_LIB)
    return HOST_SANITIZED_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
