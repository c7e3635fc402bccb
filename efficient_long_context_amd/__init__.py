"""Python binding of the ELSAA gfx950 library (libelsaa.so).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind the C ABI declared in include/elsaa.h.  PyTorch supplies device
memory and the current HIP stream.  There is no CPU fallback: if libelsaa.so is
missing or the tensors are not on a GPU, the call raises.

    import efficient_long_context_amd as elsaa
    out = elsaa.forward(q, k, v, x_gate, hyperplanes, gate_w, gate_b,
                        sort_bits=8, chunk=128, race_tables=16, race_bits=8, lam=1.0)
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libelsaa.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_DEVICE = 0, -1, -2, -3, -4
DTYPE_F32, DTYPE_BF16 = 0, 1
ABI_VERSION = 2
# elsaa_variant_t: the operator, the ablation with alpha fixed to one, and the
# two single-branch models
VARIANTS = {"full": 0, "no_alpha": 1, "race_only": 2, "sparse_only": 3}

# Every symbol include/elsaa.h declares.
EXPORTS = ("elsaa_validate", "elsaa_workspace_bytes", "elsaa_forward", "elsaa_forward_noalloc",
           "elsaa_backward_workspace_bytes", "elsaa_backward", "elsaa_status_str", "elsaa_last_error",
           "elsaa_abi_version")
NOALLOC_SCRATCH_BYTES = 64 << 20  # ELSAA_NOALLOC_SCRATCH_BYTES

AUX_FIELDS = ("sort_code_q", "sort_code_k", "race_code_q", "race_code_k", "perm_q", "perm_k",
              "race_sum", "race_cnt", "o_sparse", "lse_s", "z_lr", "alpha", "g_s", "g_lr",
              "o_lowrank")


class ElsaaAux(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in AUX_FIELDS]


class ElsaaParams(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
        ("d", ctypes.c_int32), ("d_gate", ctypes.c_int32),
        ("sort_bits", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("race_tables", ctypes.c_int32), ("race_bits", ctypes.c_int32),
        ("lambda_", ctypes.c_float), ("dtype", ctypes.c_int), ("variant", ctypes.c_int),
        ("gate_w", ctypes.c_void_p), ("gate_b", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p), ("aux", ctypes.POINTER(ElsaaAux)),
        ("stage_events", ctypes.POINTER(ctypes.c_void_p)),
        ("options", ctypes.c_uint32),
    ]

OPT_FUSED_EPILOGUE = 1  # ELSAA_OPT_FUSED_EPILOGUE
OPT_SAVE_FOR_BACKWARD = 2  # ELSAA_OPT_SAVE_FOR_BACKWARD

STAGES = ("hash", "sort", "race_build", "chunk_attention", "fuse")


class ElsaaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_str(status)}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded libelsaa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # One HIP runtime per process: PyTorch ships its own libamdhip64 (same
        # soname).  Loading torch first makes libelsaa.so bind to that copy
        # instead of pulling in a second runtime that cannot share the device.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        L.elsaa_validate.argtypes = [ctypes.POINTER(ElsaaParams)]
        L.elsaa_validate.restype = ctypes.c_int
        L.elsaa_workspace_bytes.argtypes = [ctypes.POINTER(ElsaaParams)]
        L.elsaa_workspace_bytes.restype = ctypes.c_size_t
        L.elsaa_forward.argtypes = [ctypes.c_void_p] * 5 + [ctypes.POINTER(ElsaaParams), ctypes.c_void_p]
        L.elsaa_forward.restype = ctypes.c_int
        L.elsaa_forward_noalloc.argtypes = L.elsaa_forward.argtypes
        L.elsaa_forward_noalloc.restype = ctypes.c_int
        L.elsaa_backward_workspace_bytes.argtypes = [ctypes.POINTER(ElsaaParams)]
        L.elsaa_backward_workspace_bytes.restype = ctypes.c_size_t
        L.elsaa_backward.argtypes = ([ctypes.c_void_p] * 6 + [ctypes.POINTER(ElsaaParams), ctypes.c_void_p,
                                     ctypes.c_size_t] + [ctypes.c_void_p] * 7)
        L.elsaa_backward.restype = ctypes.c_int
        L.elsaa_status_str.argtypes = [ctypes.c_int]
        L.elsaa_status_str.restype = ctypes.c_char_p
        L.elsaa_last_error.restype = ctypes.c_char_p
        L.elsaa_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().elsaa_status_str(int(status)).decode()


def last_error() -> str:
    return lib().elsaa_last_error().decode()


def make_params(B, H, N, d, d_gate, *, sort_bits, chunk, race_tables, race_bits, lam,
                dtype=DTYPE_BF16, variant=0, options=0, gate_w_ptr=0, gate_b_ptr=0, workspace_ptr=0,
                workspace_bytes=0, stream_ptr=0, aux=None, stage_events=None) -> ElsaaParams:
    p = ElsaaParams()
    p.B, p.H, p.N, p.d, p.d_gate = B, H, N, d, d_gate
    p.sort_bits, p.chunk, p.race_tables, p.race_bits = sort_bits, chunk, race_tables, race_bits
    p.lambda_ = lam
    p.dtype = dtype
    p.variant = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    p.options = int(options)
    p.gate_w, p.gate_b = gate_w_ptr or None, gate_b_ptr or None
    p.workspace, p.workspace_bytes = workspace_ptr or None, workspace_bytes
    p.stream = stream_ptr or None
    p.aux = ctypes.pointer(aux) if aux is not None else None
    p.stage_events = stage_events
    return p


def validate(params: ElsaaParams) -> int:
    return lib().elsaa_validate(ctypes.byref(params))


def workspace_bytes(params: ElsaaParams) -> int:
    return lib().elsaa_workspace_bytes(ctypes.byref(params))


def _check_tensor(name, t, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != {dtype}")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name}: must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


class Forward:
    """Reusable forward call: validates once, owns the workspace and out buffer.

    Calling the object enqueues one forward pass on torch's current stream and
    returns `out`.  With `aux=True` the per-stage outputs are also written into
    the tensors of `self.aux` (dict name -> tensor).
    """

    def __init__(self, *, B, H, N, d, d_gate=64, sort_bits, chunk, race_tables, race_bits,
                 lam=1.0, dtype="bf16", variant="full", options=0, device=None, aux=False):
        import torch
        self.torch = torch
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.dtype_code = DTYPE_BF16 if dtype == "bf16" else DTYPE_F32
        self.shape = dict(B=B, H=H, N=N, d=d, d_gate=d_gate)
        self.cfg = dict(sort_bits=sort_bits, chunk=chunk, race_tables=race_tables,
                        race_bits=race_bits, lam=float(lam), variant=variant, options=int(options))
        probe = make_params(B, H, N, d, d_gate, dtype=self.dtype_code, gate_w_ptr=1, gate_b_ptr=1,
                            **self.cfg)
        st = validate(probe)
        if st != OK:
            raise ElsaaError(st, last_error())
        self.ws_bytes = workspace_bytes(probe)
        self.workspace = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=self.device)
        self.out = torch.empty((B, H, N, d), dtype=self.tdtype, device=self.device)
        self.aux = None
        self._aux_struct = None
        if aux:
            self._make_aux()

    def _make_aux(self):
        torch = self.torch
        B, H, N, d = (self.shape[x] for x in ("B", "H", "N", "d"))
        L, P = self.cfg["race_tables"], self.cfg["race_bits"]
        cdt = torch.uint8 if P <= 8 else torch.int16
        dev = self.device
        a = {
            "sort_code_q": torch.empty((B, H, N), dtype=torch.int16, device=dev),
            "sort_code_k": torch.empty((B, H, N), dtype=torch.int16, device=dev),
            "race_code_q": torch.empty((B, H, N, L), dtype=cdt, device=dev),
            "race_code_k": torch.empty((B, H, N, L), dtype=cdt, device=dev),
            "perm_q": torch.empty((B, H, N), dtype=torch.int32, device=dev),
            "perm_k": torch.empty((B, H, N), dtype=torch.int32, device=dev),
            "race_sum": torch.empty((B, H, L, 1 << P, d), dtype=torch.float32, device=dev),
            "race_cnt": torch.empty((B, H, L, 1 << P), dtype=torch.float32, device=dev),
            "o_sparse": torch.empty((B, H, N, d), dtype=self.tdtype, device=dev),
            "lse_s": torch.empty((B, H, N), dtype=torch.float32, device=dev),
            "z_lr": torch.empty((B, H, N), dtype=torch.float32, device=dev),
            "alpha": torch.empty((B, H, N), dtype=torch.float32, device=dev),
            "g_s": torch.empty((B, H, N), dtype=torch.float32, device=dev),
            "g_lr": torch.empty((B, H, N), dtype=torch.float32, device=dev),
            "o_lowrank": torch.empty((B, H, N, d), dtype=torch.float32, device=dev),
        }
        self.aux = a
        s = ElsaaAux()
        for name in AUX_FIELDS:
            setattr(s, name, a[name].data_ptr())
        self._aux_struct = s

    def __call__(self, q, k, v, x_gate, hyperplanes, gate_w, gate_b, stream=None,
                 stage_events=None):
        """stage_events: optional ctypes array of 10 hipEvent_t handles, a (begin,
        end) pair per stage in STAGES order (see elsaa.h)."""
        torch = self.torch
        B, H, N, d, dg = (self.shape[x] for x in ("B", "H", "N", "d", "d_gate"))
        R = self.cfg["sort_bits"] + self.cfg["race_tables"] * self.cfg["race_bits"]
        dev, dt = self.device, self.tdtype
        _check_tensor("q", q, (B, H, N, d), dt, dev)
        _check_tensor("k", k, (B, H, N, d), dt, dev)
        _check_tensor("v", v, (B, H, N, d), dt, dev)
        _check_tensor("x_gate", x_gate, (B, N, dg), dt, dev)
        _check_tensor("hyperplanes", hyperplanes, (R, d), dt, dev)
        _check_tensor("gate_w", gate_w, (2, H, dg), torch.float32, dev)
        _check_tensor("gate_b", gate_b, (2, H), torch.float32, dev)
        if stream is None:
            stream = torch.cuda.current_stream(dev)
        p = make_params(B, H, N, d, dg, dtype=self.dtype_code, gate_w_ptr=gate_w.data_ptr(),
                        gate_b_ptr=gate_b.data_ptr(), workspace_ptr=self.workspace.data_ptr(),
                        workspace_bytes=self.ws_bytes, stream_ptr=stream.cuda_stream,
                        aux=self._aux_struct, stage_events=stage_events, **self.cfg)
        st = lib().elsaa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), x_gate.data_ptr(),
                                 hyperplanes.data_ptr() if R else None, ctypes.byref(p),
                                 self.out.data_ptr())
        if st != OK:
            raise ElsaaError(st, last_error())
        return self.out


class Backward:
    """Backward pass of a Forward object's last call (its workspace holds that
    call's results).  Owns the backward scratch and the gradient tensors;
    calling it enqueues elsaa_backward on torch's current stream and returns
    (dq, dk, dv, dx_gate, dgate_w, dgate_b, dlambda) as tensors."""

    def __init__(self, fwd: "Forward"):
        torch = fwd.torch
        self.fwd = fwd
        B, H, N, d, dg = (fwd.shape[x] for x in ("B", "H", "N", "d", "d_gate"))
        probe = make_params(B, H, N, d, dg, dtype=fwd.dtype_code, gate_w_ptr=1, gate_b_ptr=1, **fwd.cfg)
        self.ws_bytes = lib().elsaa_backward_workspace_bytes(ctypes.byref(probe))
        if self.ws_bytes == 0:
            raise ElsaaError(ERR_UNSUPPORTED, last_error())
        dev, dt = fwd.device, fwd.tdtype
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.dq = torch.empty((B, H, N, d), dtype=dt, device=dev)
        self.dk = torch.empty_like(self.dq)
        self.dv = torch.empty_like(self.dq)
        self.dx_gate = torch.empty((B, N, dg), dtype=dt, device=dev)
        self.dgate_w = torch.empty((2, H, dg), dtype=torch.float32, device=dev)
        self.dgate_b = torch.empty((2, H), dtype=torch.float32, device=dev)
        self.dlambda = torch.empty((1,), dtype=torch.float32, device=dev)

    def __call__(self, q, k, v, x_gate, gate_w, gate_b, dy, stream=None):
        f = self.fwd
        torch = f.torch
        B, H, N, d, dg = (f.shape[x] for x in ("B", "H", "N", "d", "d_gate"))
        _check_tensor("dy", dy, (B, H, N, d), f.tdtype, f.device)
        if stream is None:
            stream = torch.cuda.current_stream(f.device)
        p = make_params(B, H, N, d, dg, dtype=f.dtype_code, gate_w_ptr=gate_w.data_ptr(),
                        gate_b_ptr=gate_b.data_ptr(), workspace_ptr=f.workspace.data_ptr(),
                        workspace_bytes=f.ws_bytes, stream_ptr=stream.cuda_stream, **f.cfg)
        st = lib().elsaa_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), x_gate.data_ptr(),
                                  f.out.data_ptr(), dy.data_ptr(), ctypes.byref(p),
                                  self.workspace.data_ptr(), self.ws_bytes, self.dq.data_ptr(),
                                  self.dk.data_ptr(), self.dv.data_ptr(), self.dx_gate.data_ptr(),
                                  self.dgate_w.data_ptr(), self.dgate_b.data_ptr(),
                                  self.dlambda.data_ptr())
        if st != OK:
            raise ElsaaError(st, last_error())
        return (self.dq, self.dk, self.dv, self.dx_gate, self.dgate_w, self.dgate_b, self.dlambda)


def forward(q, k, v, x_gate, hyperplanes, gate_w, gate_b, *, sort_bits, chunk, race_tables,
            race_bits, lam=1.0, variant="full", aux=False):
    """One-shot forward pass (allocates workspace and output)."""
    import torch
    B, H, N, d = q.shape
    dtype = "bf16" if q.dtype == torch.bfloat16 else "fp32"
    f = Forward(B=B, H=H, N=N, d=d, d_gate=x_gate.shape[-1], sort_bits=sort_bits, chunk=chunk,
                race_tables=race_tables, race_bits=race_bits, lam=lam, dtype=dtype,
                variant=variant, device=q.device, aux=aux)
    out = f(q, k, v, x_gate, hyperplanes, gate_w, gate_b)
    return (out, f.aux) if aux else out
