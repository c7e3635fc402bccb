"""Host-only tests of the C ABI: the library loads, exports every function
include/elsaa.h declares, and validates every argument before touching the GPU.
No compute call is made (there is no GPU here); every elsaa_forward call below
fails validation and returns before any launch."""
import ctypes
import os
import re

import pytest

import efficient_long_context_amd as elsaa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "elsaa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(elsaa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = elsaa.lib()
    names = header_functions()
    assert set(names) == set(elsaa.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name
    assert lib.elsaa_abi_version() == elsaa.ABI_VERSION == 2


def test_status_strings():
    assert elsaa.status_str(0) == "ELSAA_OK"
    assert elsaa.status_str(-1) == "ELSAA_ERR_INVALID_ARG"
    assert elsaa.status_str(-2) == "ELSAA_ERR_UNSUPPORTED"
    assert elsaa.status_str(-3) == "ELSAA_ERR_WORKSPACE"
    assert elsaa.status_str(-4) == "ELSAA_ERR_DEVICE"
    assert elsaa.status_str(7) == "ELSAA_ERR_UNKNOWN"


def params(**over):
    kw = dict(B=2, H=12, N=32768, d=64, d_gate=64, sort_bits=8, chunk=128, race_tables=16,
              race_bits=8, lam=1.0, gate_w_ptr=0x1000, gate_b_ptr=0x2000)
    kw.update(over)
    B, H, N, d, dg = (kw.pop(x) for x in ("B", "H", "N", "d", "d_gate"))
    return elsaa.make_params(B, H, N, d, dg, **kw)


def test_valid_params_and_workspace_size():
    p = params()
    assert elsaa.validate(p) == elsaa.OK
    ws = elsaa.workspace_bytes(p)
    rows = 2 * 12 * 32768
    # codes + perms + tables (bf16 sums, binary32 counts) at least
    tables = 24 * 16 * 256 * (64 * 2 + 4)
    base = 2 * rows * 2 + 2 * rows * 16 + 2 * rows * 4 + tables
    # the separate fusion kernel reads o_s and its LSE back; with the fused
    # epilogue neither goes to memory
    assert ws >= base + rows * 64 * 2 + rows * 4
    fused = elsaa.workspace_bytes(params(options=elsaa.OPT_FUSED_EPILOGUE))
    assert base <= fused < base + rows * 64 * 2
    # saving for the backward adds o_lr (dtype) and three floats per token-head,
    # and excludes the fused epilogue
    saved = elsaa.workspace_bytes(params(options=elsaa.OPT_SAVE_FOR_BACKWARD))
    assert ws + rows * (64 * 2 + 12) <= saved <= ws + rows * (64 * 2 + 12) + 4 * 256
    both = elsaa.workspace_bytes(params(options=elsaa.OPT_SAVE_FOR_BACKWARD | elsaa.OPT_FUSED_EPILOGUE))
    assert both == saved
    # where the fused epilogue does not apply (12 tables) the option is ignored
    assert (elsaa.workspace_bytes(params(race_tables=12, options=elsaa.OPT_FUSED_EPILOGUE))
            == elsaa.workspace_bytes(params(race_tables=12)))
    assert ws < 400 * 2 ** 20


@pytest.mark.parametrize("over,status", [
    (dict(N=1000), elsaa.ERR_INVALID_ARG),            # chunk does not divide N
    (dict(B=0), elsaa.ERR_INVALID_ARG),
    (dict(H=-1), elsaa.ERR_INVALID_ARG),
    (dict(lam=-1.0), elsaa.ERR_INVALID_ARG),
    (dict(lam=float("nan")), elsaa.ERR_INVALID_ARG),
    (dict(lam=float("inf")), elsaa.ERR_INVALID_ARG),
    (dict(race_tables=0), elsaa.ERR_INVALID_ARG),
    (dict(sort_bits=-1), elsaa.ERR_INVALID_ARG),
    (dict(gate_w_ptr=0), elsaa.ERR_INVALID_ARG),
    (dict(dtype=5), elsaa.ERR_INVALID_ARG),
    (dict(d=96), elsaa.ERR_UNSUPPORTED),
    (dict(sort_bits=13), elsaa.ERR_UNSUPPORTED),
    (dict(race_bits=13), elsaa.ERR_UNSUPPORTED),
    (dict(race_tables=65), elsaa.ERR_UNSUPPORTED),
    (dict(race_tables=32, race_bits=10), elsaa.ERR_UNSUPPORTED),  # 32 * 1024 > 16384
    (dict(chunk=96, N=96 * 300), elsaa.ERR_UNSUPPORTED),
    (dict(d_gate=1024), elsaa.ERR_UNSUPPORTED),
    (dict(variant=4), elsaa.ERR_INVALID_ARG),
    (dict(variant=-1), elsaa.ERR_INVALID_ARG),
    (dict(options=4), elsaa.ERR_INVALID_ARG),
    # per-(b, h) byte extents at 2^31 and beyond: the kernels' 32-bit offsets
    (dict(B=1, H=1, d=128, N=1 << 24), elsaa.ERR_UNSUPPORTED),                    # bf16, 2^32 B
    (dict(B=1, H=1, d=128, N=1 << 23), elsaa.ERR_UNSUPPORTED),                    # bf16, 2^31 B
    (dict(B=1, H=1, d=128, N=1 << 22, dtype=elsaa.DTYPE_F32), elsaa.ERR_UNSUPPORTED),  # fp32 d=128
    (dict(B=1, H=1, d=64, N=1 << 23, dtype=elsaa.DTYPE_F32), elsaa.ERR_UNSUPPORTED),   # fp32 d=64
    (dict(B=1, H=1, d_gate=512, N=1 << 20, dtype=elsaa.DTYPE_F32), elsaa.ERR_UNSUPPORTED),  # x_gate
])
def test_invalid_params_rejected(over, status):
    p = params(**over)
    assert elsaa.validate(p) == status
    assert elsaa.workspace_bytes(p) == 0
    assert elsaa.last_error() != ""


@pytest.mark.parametrize("over", [
    dict(B=1, H=1, d=128, N=(1 << 23) - 128),                       # bf16 d=128 just below 2^31 B
    dict(B=1, H=1, d=128, N=(1 << 22) - 128, dtype=elsaa.DTYPE_F32),
    dict(B=1, H=1, d=64, N=(1 << 23) - 128, dtype=elsaa.DTYPE_F32),
    dict(sort_bits=0, race_bits=0),                                   # no hyperplanes at all
    dict(variant=1), dict(variant=2), dict(variant=3),
])
def test_valid_edge_params(over):
    p = params(**over)
    assert elsaa.validate(p) == elsaa.OK, elsaa.last_error()
    assert elsaa.workspace_bytes(p) > 0


def test_forward_accepts_null_planes_without_planes():
    """sort_bits = race_bits = 0: no hyperplane rows, so a NULL pointer passes the
    pointer checks (the call then stops at the missing workspace, before any launch)."""
    lib = elsaa.lib()
    fake = ctypes.c_void_p(0x10000)
    p = params(sort_bits=0, race_bits=0)
    assert lib.elsaa_forward(fake, fake, fake, fake, None, ctypes.byref(p), fake) == elsaa.ERR_WORKSPACE
    p = params()
    assert lib.elsaa_forward(fake, fake, fake, fake, None, ctypes.byref(p), fake) == elsaa.ERR_INVALID_ARG


def test_forward_rejects_before_launch():
    lib = elsaa.lib()
    fake = ctypes.c_void_p(0x10000)
    # invalid params
    p = params(N=1000)
    assert lib.elsaa_forward(fake, fake, fake, fake, fake, ctypes.byref(p), fake) == elsaa.ERR_INVALID_ARG
    # null tensor
    p = params()
    assert lib.elsaa_forward(None, fake, fake, fake, fake, ctypes.byref(p), fake) == elsaa.ERR_INVALID_ARG
    # missing / short workspace
    assert lib.elsaa_forward(fake, fake, fake, fake, fake, ctypes.byref(p), fake) == elsaa.ERR_WORKSPACE
    need = elsaa.workspace_bytes(p)
    p = params(workspace_ptr=0x20000, workspace_bytes=need - 1)
    assert lib.elsaa_forward(fake, fake, fake, fake, fake, ctypes.byref(p), fake) == elsaa.ERR_WORKSPACE
    assert "workspace" in elsaa.last_error()
    assert lib.elsaa_forward(fake, fake, fake, fake, fake, None, fake) == elsaa.ERR_INVALID_ARG


def test_backward_validation_before_any_device_call():
    lib = elsaa.lib()
    fake = ctypes.c_void_p(0x10000)
    f32 = ctypes.c_void_p(0x30000)
    p = params()
    assert elsaa.lib().elsaa_backward_workspace_bytes(ctypes.byref(p)) > 0
    # the fused epilogue keeps o_s and the LSE out of memory: no backward
    pf = params(options=elsaa.OPT_FUSED_EPILOGUE)
    assert lib.elsaa_backward_workspace_bytes(ctypes.byref(pf)) == 0
    args = [fake] * 6 + [None, fake, 1 << 30] + [fake] * 4 + [f32] * 3
    args[6] = ctypes.byref(pf)
    assert lib.elsaa_backward(*args) == elsaa.ERR_UNSUPPORTED
    # missing forward workspace, then missing backward workspace
    args[6] = ctypes.byref(p)
    assert lib.elsaa_backward(*args) == elsaa.ERR_WORKSPACE
    need = elsaa.workspace_bytes(p)
    pw = params(workspace_ptr=0x20000, workspace_bytes=need)
    args[6] = ctypes.byref(pw)
    args[7], args[8] = None, 0
    assert lib.elsaa_backward(*args) == elsaa.ERR_WORKSPACE
    assert "backward workspace" in elsaa.last_error()
    # a NULL gradient pointer
    args[7], args[8] = fake, 1 << 40
    args[9] = None
    assert lib.elsaa_backward(*args) == elsaa.ERR_INVALID_ARG


def test_noalloc_rejects_problems_above_its_scratch_before_any_device_call():
    """elsaa_forward_noalloc ignores the workspace fields and rejects a problem
    whose scratch exceeds its fixed array on the host, before touching the
    device (there is none here)."""
    lib = elsaa.lib()
    fake = ctypes.c_void_p(0x10000)
    p = params()  # the 32K-token text shape: far above 64 MiB of scratch
    assert elsaa.workspace_bytes(p) > elsaa.NOALLOC_SCRATCH_BYTES
    assert lib.elsaa_forward_noalloc(fake, fake, fake, fake, fake, ctypes.byref(p), fake) == elsaa.ERR_WORKSPACE
    assert "noalloc" in elsaa.last_error()
    p = params(N=1000)
    assert lib.elsaa_forward_noalloc(fake, fake, fake, fake, fake, ctypes.byref(p), fake) == elsaa.ERR_INVALID_ARG
    p = params(B=1, H=1, N=4096)
    assert elsaa.workspace_bytes(p) <= elsaa.NOALLOC_SCRATCH_BYTES
    assert lib.elsaa_forward_noalloc(None, fake, fake, fake, fake, ctypes.byref(p), fake) == elsaa.ERR_INVALID_ARG


def test_forward_rejects_misaligned_pointers():
    lib = elsaa.lib()
    fake = ctypes.c_void_p(0x10000)
    need = elsaa.workspace_bytes(params())
    p = params(workspace_ptr=0x20000, workspace_bytes=need)
    odd = ctypes.c_void_p(0x10008)  # 8-byte aligned only
    for i in range(6):
        args = [fake] * 6
        args[i] = odd
        q, k, v, x, planes, out = args
        assert lib.elsaa_forward(q, k, v, x, planes, ctypes.byref(p), out) == elsaa.ERR_INVALID_ARG
        assert "16-byte" in elsaa.last_error()
    p = params(workspace_ptr=0x20080, workspace_bytes=need)  # 128-byte aligned only
    assert lib.elsaa_forward(fake, fake, fake, fake, fake, ctypes.byref(p), fake) == elsaa.ERR_WORKSPACE
    assert "256-byte" in elsaa.last_error()


def test_struct_layout_matches_header():
    # elsaa_params_t: 9 int32, float, two enums (dtype, variant), then 8-byte
    # aligned pointers
    assert ctypes.sizeof(elsaa.ElsaaParams) == 48 + 8 * 2 + 8 + 8 + 8 + 8 + 8 + 8
    assert elsaa.ElsaaParams.variant.offset == 44
    assert elsaa.ElsaaParams.gate_w.offset == 48
    assert elsaa.ElsaaParams.options.offset == 48 + 8 * 7
    assert ctypes.sizeof(elsaa.ElsaaAux) == 15 * 8
