"""Builds libdsa.so in-tree with hipcc for gfx950.

``python -m sparse_attention_18_amd.build`` (or ``build_library()``) compiles
every HIP source under ``csrc/`` and links them, with the C-ABI layer, into
``sparse_attention_18_amd/libdsa.so``.  The build runs without a GPU (hipcc
cross-compiles the device code).

Two variants share the kernel objects and differ only in the C-ABI layer:
* ``libdsa_debug.so`` (always built): abi.cpp with ``DSA_DEBUG``, which
  copies the device offset arrays and block tables of every call to the host
  and checks them before launching (include/dsa.h, "Debug builds");
* ``libdsa_asan.so`` (``build_asan_library()``, for the CPU tests): abi.cpp's
  host code built with AddressSanitizer; it is loaded with the sanitizer's
  runtime preloaded.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdsa.so")
ROOT = os.path.dirname(PKG)

ARCH = "gfx950"
SOURCES = ["indexer.hip", "topk.hip", "sparse_attn.hip", "prefill_mha.hip", "align.hip", "indexer_bwd.hip",
           "abi.cpp"]
# Packed-FP32 VALU forms are kept out of every device code object.
# IEEE mode is off (no NaN quieting on min/max): the kernels never rely on
# signalling-NaN behaviour, and fmaxf then lowers to a single v_max_f32.
FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mno-amdgpu-ieee", "-fno-honor-nans",
         "-Wno-unused-command-line-argument", f"-I{os.path.join(ROOT, 'include')}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdsa.so)")


def _compile(src: str, verbose: bool, suffix: str = "", extra=()) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + suffix + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc()] + lang + FLAGS + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    return obj


LIB_DEBUG = os.path.join(PKG, "libdsa_debug.so")
LIB_ASAN = os.path.join(BUILD, "libdsa_asan.so")
# The sanitizer applies to host code only (the device code is unchanged).
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _link(path: str, objs, extra=(), verbose=False) -> str:
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + list(extra) + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(path)} failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)
    return path


def _kernel_objects():
    return [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "abi.cpp"]


def build_library(verbose: bool = False) -> str:
    """Compile and link libdsa.so and libdsa_debug.so; returns libdsa.so's
    path.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, "", ()) for s in SOURCES] + [("abi.cpp", "_debug", ("-DDSA_DEBUG",))]
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1], j[2]), jobs))
    kernels = _kernel_objects()
    _link(LIB_DEBUG, kernels + [objs[-1]], verbose=verbose)
    return _link(LIB, objs[:-1], verbose=verbose)


def build_asan_library(verbose: bool = False) -> str:
    """libdsa_asan.so: the kernel objects of the last build_library() with
    abi.cpp's host code under AddressSanitizer.  Load it only with the
    sanitizer runtime (asan_runtime()) preloaded."""
    if not all(os.path.exists(o) for o in _kernel_objects()):
        build_library(verbose)
    obj = _compile("abi.cpp", verbose, "_asan", tuple(ASAN_FLAGS))
    return _link(LIB_ASAN, _kernel_objects() + [obj], ASAN_FLAGS + ["-shared-libasan"], verbose)


def asan_runtime() -> str:
    """The compiler's AddressSanitizer runtime library (to preload)."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found next to hipcc's clang")
    return path


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
