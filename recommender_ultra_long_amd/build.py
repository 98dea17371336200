"""Builds libsa.so (the HIP kernels and the C-ABI of include/sa.h) in-tree.

Every source is compiled for gfx950 with hipcc and linked into
recommender_ultra_long_amd/libsa.so.  Object files go to _build/ at the
repository root.  Packed fp32 instructions are disabled for all device code.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsa.so")

SOURCES = ["sa_api.cpp", "sa_block_api.cpp", "sa_action_api.cpp", "sa_action.hip",
           "sa_stca_api.cpp", "sa_stca.hip", "sa_gemm_mx.hip", "sa_fwd_bf16.hip", "sa_fused_bf16.hip", "sa_fwd_f32.hip", "sa_reduce.hip", "sa_tok.hip",
           "sa_bwd.hip", "sa_fold.hip", "sa_block.hip"]

COMMON = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src, hipcc):
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc, *COMMON, "-I", CSRC, "-I", os.path.join(ROOT, "include"), "-c",
           os.path.join(CSRC, src), "-o", out]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out


def _objects_for(sources):
    return [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in sources]


def build_host_asan(verbose=False) -> str:
    """A copy of the library whose host code (the C-ABI layer: argument
    validation, plans, workspace layout) is built with AddressSanitizer, for
    CPU-only checks of the validation paths.  Device code is unchanged (the
    kernel objects of ``build``); the sanitizer applies to the host pass only.
    The library leaves the sanitizer's runtime unresolved: load it into a
    process started with that runtime preloaded (``asan_runtime()``)."""
    if not all(os.path.exists(o) for o in _objects_for(SOURCES)):
        build(verbose)
    hipcc = _hipcc()
    out_dir = os.path.join(BUILD, "asan")
    os.makedirs(out_dir, exist_ok=True)
    api = [s for s in SOURCES if s.endswith(".cpp")]
    objs = []
    for src in api:
        out = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
               "-Wno-unused-command-line-argument", "-I", CSRC, "-I", os.path.join(ROOT, "include"),
               "-c", os.path.join(CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        objs.append(out)
    lib = os.path.join(out_dir, "libsa_asan.so")
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, *objs,
           *_objects_for([s for s in SOURCES if not s.endswith(".cpp")])]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print("built", lib)
    return lib


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found")
    return path


def build(verbose=False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
