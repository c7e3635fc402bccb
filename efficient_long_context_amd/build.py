"""Build the ELSAA gfx950 library (libelsaa.so) in-tree with hipcc.

Every HIP source under csrc/ is compiled for gfx950 only, with packed-FP32
instruction selection disabled, into _build/, then linked into
efficient_long_context_amd/libelsaa.so next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libelsaa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


# Per-source extra flags.  The hash and the backward kernels read every MFMA
# result with plain VALU instructions; their accumulators are kept in VGPRs
# (no AGPR copies; the backward's dq kernel then fits four waves per SIMD).
EXTRA: dict = {"k1_hash.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "k6_backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


# Host-code sanitizers: AddressSanitizer and UBSan on the host side of every
# source (each -fsanitize= behind -Xarch_host, so no device code is
# instrumented), linked against the shared sanitizer runtime, which the
# process must preload.  For host-only tests; the library behaves the same.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
CLANGXX = os.environ.get("CLANGXX", "/opt/rocm/llvm/bin/clang++")


def build_sanitized(out_dir: str, jobs: int = 8) -> str:
    """Build a host-sanitized copy of the library into out_dir; returns its path."""
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir, SANITIZE), srcs))
    lib = os.path.join(out_dir, "libelsaa_sanitized.so")
    cmd = [CLANGXX, "-shared", "-shared-libsan", "-fsanitize=address,undefined", *objs,
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stdout}\n{r.stderr}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
