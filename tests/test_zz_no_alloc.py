"""The allocation-free entry point against the workspace one.

elsaa_forward_noalloc runs the same kernels as elsaa_forward with its scratch
in a fixed device array instead of a caller workspace.  Two calls in a row
(the second on a smaller problem, so it runs over the first call's leftover
scratch contents) must reproduce elsaa_forward's outputs: codes,
permutations and counts bit for bit, and every floating output within the
parity tolerance (the kernels are the same, so in practice bit for bit too).
"""
import ctypes

import numpy as np
import pytest

import workloads
from gpu_common import TOL, rel_err, to_device

pytestmark = pytest.mark.gpu


def _run(inp, noalloc: bool):
    import torch

    import efficient_long_context_amd as elsaa
    wl = inp.wl
    dev = torch.device("cuda", 0)
    x = to_device(inp, dev)
    f = elsaa.Forward(B=wl.B, H=wl.H, N=wl.N, d=wl.d, d_gate=wl.d_gate, sort_bits=wl.sort_bits,
                      chunk=wl.chunk, race_tables=wl.race_tables, race_bits=wl.race_bits, lam=wl.lam,
                      dtype=wl.dtype, device=dev, aux=True)
    if not noalloc:
        out = f(x["q"], x["k"], x["v"], x["x_gate"], x["hyperplanes"], x["gate_w"], x["gate_b"])
    else:
        out = torch.empty_like(f.out)
        stream = torch.cuda.current_stream(dev)
        p = elsaa.make_params(wl.B, wl.H, wl.N, wl.d, wl.d_gate, sort_bits=wl.sort_bits, chunk=wl.chunk,
                              race_tables=wl.race_tables, race_bits=wl.race_bits, lam=wl.lam,
                              dtype=elsaa.DTYPE_BF16 if wl.dtype == "bf16" else elsaa.DTYPE_F32,
                              gate_w_ptr=x["gate_w"].data_ptr(), gate_b_ptr=x["gate_b"].data_ptr(),
                              stream_ptr=stream.cuda_stream, aux=f._aux_struct)
        st = elsaa.lib().elsaa_forward_noalloc(x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(),
                                               x["x_gate"].data_ptr(), x["hyperplanes"].data_ptr(),
                                               ctypes.byref(p), out.data_ptr())
        assert st == elsaa.OK, elsaa.last_error()
    torch.cuda.synchronize()
    res = {"y": out.float().cpu().numpy()}
    for name, t in f.aux.items():
        res[name] = t.float().cpu().numpy() if t.is_floating_point() else t.cpu().numpy()
    return res


@pytest.mark.parametrize("first,second", [
    (("text32k-bf16", dict(B=1, H=2, N=8192)), ("text32k-bf16", dict(B=1, H=1, N=2048))),
    (("needle256k-bf16", dict(H=2, N=8192)), ("small-bf16", dict(B=1, H=2, N=1024))),
    (("tiny-fp32", dict(H=2)), ("tiny-fp32", dict(N=512, chunk=64))),
    # a RACE build in two token blocks (46 MB of scratch), then one block
    (("needle256k-bf16", dict(H=1, N=65536, chunk=64)), ("needle256k-bf16", dict(H=1, N=4096))),
])
def test_noalloc_matches_workspace_entry_point(first, second):
    for name, over in (first, second):
        wl = workloads.workload(name, **over)
        inp = workloads.generate(wl, seed=17)
        print(f"[noalloc] {name} {over}", flush=True)
        ref = _run(inp, noalloc=False)
        got = _run(inp, noalloc=True)
        for key in ("sort_code_q", "sort_code_k", "race_code_q", "race_code_k", "perm_q", "perm_k",
                    "race_cnt"):
            np.testing.assert_array_equal(got[key], ref[key], err_msg=f"{name} {key}")
        tol = TOL[wl.dtype]
        for key in ("y", "race_sum", "o_sparse", "lse_s", "z_lr", "alpha", "g_s", "g_lr", "o_lowrank"):
            assert rel_err(got[key], ref[key]) <= tol, f"{name} {key}"
        np.testing.assert_array_equal(got["y"], ref["y"], err_msg=f"{name} y (same kernels)")
