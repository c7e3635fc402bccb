"""Host code under AddressSanitizer and UBSan (CPU only, no device calls).

  * The oracle, built by gcc with -fsanitize=address,undefined, runs its pin
    tests in a child process with the gcc sanitizer runtime preloaded.
  * The HIP library, its host side built with the same sanitizers (device code
    untouched), runs every host-only path of the C ABI -- validation,
    workspace sizes and the rejection paths of the forward, allocation-free
    forward and backward entry points -- in a child process with the clang
    runtime preloaded.
Any sanitizer report fails the child (UBSan is made fatal), and the child's
exit status fails the test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ENV_BASE = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _gcc_runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_under_asan_ubsan(tmp_path):
    import oracle
    asan = _gcc_runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc AddressSanitizer runtime not installed")
    lib = str(tmp_path / "liboracle_sanitized.so")
    cmd = ["gcc", *oracle.CFLAGS, "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", oracle._SRC, "-o", lib, "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(ENV_BASE, LD_PRELOAD=asan, ELSAA_ORACLE_LIB=lib, OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py", "tests/test_oracle_backward_pins.py",
                        "-k", "not autograd"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


HOST_PATHS = r'''
import ctypes, sys
sys.path.insert(0, ".")
import efficient_long_context_amd as elsaa
from efficient_long_context_amd import ElsaaParams, make_params
L = ctypes.CDLL(sys.argv[1])
P = ctypes.POINTER(ElsaaParams)
L.elsaa_validate.argtypes = [P]
L.elsaa_workspace_bytes.argtypes = [P]; L.elsaa_workspace_bytes.restype = ctypes.c_size_t
L.elsaa_backward_workspace_bytes.argtypes = [P]; L.elsaa_backward_workspace_bytes.restype = ctypes.c_size_t
L.elsaa_forward.argtypes = [ctypes.c_void_p] * 5 + [P, ctypes.c_void_p]
L.elsaa_forward_noalloc.argtypes = L.elsaa_forward.argtypes
L.elsaa_backward.argtypes = [ctypes.c_void_p] * 6 + [P, ctypes.c_void_p, ctypes.c_size_t] + [ctypes.c_void_p] * 7
L.elsaa_status_str.restype = ctypes.c_char_p
L.elsaa_last_error.restype = ctypes.c_char_p
base = dict(B=2, H=12, N=32768, d=64, d_gate=64, sort_bits=8, chunk=128, race_tables=16, race_bits=8, lam=1.0,
            gate_w_ptr=0x1000, gate_b_ptr=0x2000)
def params(**over):
    kw = dict(base); kw.update(over)
    B, H, N, d, dg = (kw.pop(x) for x in ("B", "H", "N", "d", "d_gate"))
    return make_params(B, H, N, d, dg, **kw)
cases = [{}, dict(N=1000), dict(B=0), dict(lam=-1.0), dict(lam=float("nan")), dict(race_tables=0),
         dict(sort_bits=-1), dict(gate_w_ptr=0), dict(dtype=5), dict(d=96), dict(sort_bits=13),
         dict(race_bits=13), dict(race_tables=65), dict(race_tables=32, race_bits=10), dict(chunk=96, N=96 * 300),
         dict(d_gate=1024), dict(variant=4), dict(options=4), dict(B=1, H=1, d=128, N=1 << 23),
         dict(sort_bits=0, race_bits=0), dict(variant=2), dict(variant=3), dict(options=1), dict(options=2),
         dict(dtype=0, d=128, N=4096, chunk=64), dict(race_tables=3, race_bits=12, sort_bits=12)]
for c in cases:
    p = params(**c)
    L.elsaa_validate(ctypes.byref(p)); L.elsaa_workspace_bytes(ctypes.byref(p))
    L.elsaa_backward_workspace_bytes(ctypes.byref(p)); L.elsaa_last_error()
fake, f32 = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x30000)
for c in cases[:8]:
    p = params(**c)
    L.elsaa_forward(fake, fake, fake, fake, fake, ctypes.byref(p), fake)
    L.elsaa_forward_noalloc(fake, fake, fake, fake, fake, ctypes.byref(p), fake)
    L.elsaa_backward(fake, fake, fake, fake, fake, fake, ctypes.byref(p), None, 0, fake, fake, fake, fake, f32, f32, f32)
p = params()
assert L.elsaa_forward(None, fake, fake, fake, fake, ctypes.byref(p), fake) == elsaa.ERR_INVALID_ARG
assert L.elsaa_forward(fake, fake, fake, fake, fake, None, fake) == elsaa.ERR_INVALID_ARG
assert L.elsaa_forward(fake, fake, fake, fake, fake, ctypes.byref(p), fake) == elsaa.ERR_WORKSPACE
pw = params(workspace_ptr=0x20000, workspace_bytes=L.elsaa_workspace_bytes(ctypes.byref(p)) - 1)
assert L.elsaa_forward(fake, fake, fake, fake, fake, ctypes.byref(pw), fake) == elsaa.ERR_WORKSPACE
assert L.elsaa_forward_noalloc(fake, fake, fake, fake, fake, ctypes.byref(p), fake) == elsaa.ERR_WORKSPACE
for s in range(-6, 2):
    L.elsaa_status_str(s)
print("host paths ok")
'''


def test_host_library_under_asan_ubsan(tmp_path):
    from efficient_long_context_amd import build as hip_build
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang AddressSanitizer runtime not installed")
    lib = hip_build.build_sanitized(str(tmp_path / "san"))
    env = dict(ENV_BASE, LD_PRELOAD=rt[-1])
    r = subprocess.run([sys.executable, "-c", HOST_PATHS, lib], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "host paths ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
