"""GPU parity of the backward pass: elsaa_backward through the C ABI against the
oracle's exact gradients (tests/test_oracle_backward_pins.py pins those to
finite differences).  Every gradient -- dq, dk, dv, dx_gate, dW_g, db_g and
dlambda -- must satisfy max|d| / max|ref| <= 2e-2 (bfloat16 inputs) or 1e-4
(binary32), per tensor; two calls must agree bit for bit.
"""
import numpy as np
import pytest

import workloads
from gpu_common import TOL, rel_err, to_device

pytestmark = pytest.mark.gpu

CASES = {
    "tiny-fp32": ("tiny-fp32", {}, "full"),
    "fp32-d128-w128": ("tiny-fp32", dict(d=128, H=2, N=2048, chunk=128), "full"),
    "small-bf16-w64": ("small-bf16", dict(B=1, H=2, N=2048), "full"),
    "text32k-w128": ("text32k-bf16", dict(B=1, H=2, N=4096), "full"),
    "needle-d128-w256": ("needle256k-bf16", dict(H=2, N=4096), "full"),
    "text32k-ns0": ("text32k-bf16", dict(B=1, H=2, N=4096, sort_bits=0), "full"),
    "small-P12-L4": ("small-bf16", dict(B=1, H=2, N=2048, race_tables=4, race_bits=12), "full"),
    "small-L3-dgate48": ("small-bf16", dict(B=2, H=2, N=1024, race_tables=3, d_gate=48), "full"),
    "text32k-no-alpha": ("text32k-bf16", dict(B=1, H=2, N=4096), "no_alpha"),
    "text32k-race-only": ("text32k-bf16", dict(B=1, H=2, N=4096), "race_only"),
    "text32k-sparse-only": ("text32k-bf16", dict(B=1, H=2, N=4096), "sparse_only"),
    "fp32-race-only": ("tiny-fp32", dict(H=2), "race_only"),
    "fp32-sparse-only": ("tiny-fp32", dict(H=2), "sparse_only"),
    # segments longer than 65536: 32-bit permutation indices and the tiled rank
    # of the RACE transposes
    "small-long-N": ("small-bf16", dict(B=1, H=1, N=65536 + 192, chunk=64), "full"),
    # a forward in two token blocks (d = 128, 16 MB of value rows a head) and
    # a backward whose query-side ranks need one workgroup a CU (2^10 buckets,
    # 65536 16-bit indices), on the RACE branch those two change.  (The full
    # model at this size puts d gate_b, a two-element sum over 65536 tokens,
    # at 2.1e-2 of its maximum with and without token blocks.)
    "needle-race-blocks": ("needle256k-bf16", dict(H=1, N=65536, chunk=64), "race_only"),
}
# the same with the forward keeping o_lr, the counts and the gates for the
# backward (ELSAA_OPT_SAVE_FOR_BACKWARD)
SAVED = ("tiny-fp32", "small-bf16-w64", "text32k-w128", "needle-d128-w256", "small-L3-dgate48",
         "text32k-no-alpha", "text32k-race-only", "needle-race-blocks")


def _dy(inp, seed):
    rng = np.random.default_rng(seed)
    d64 = rng.standard_normal(inp.q.shape)
    if inp.wl.dtype == "bf16":
        bits = workloads.round_to_bf16_bits(d64)
        return workloads.bf16_bits_to_f32(bits), bits
    return d64.astype(np.float32), None


def run_backward(inp, dy, dy_bits, variant, repeat=1, options=0):
    import torch

    import efficient_long_context_amd as elsaa
    wl = inp.wl
    dev = torch.device("cuda", 0)
    x = to_device(inp, dev)
    f = elsaa.Forward(B=wl.B, H=wl.H, N=wl.N, d=wl.d, d_gate=wl.d_gate, sort_bits=wl.sort_bits,
                      chunk=wl.chunk, race_tables=wl.race_tables, race_bits=wl.race_bits, lam=wl.lam,
                      dtype=wl.dtype, variant=variant, options=options, device=dev)
    bwd = elsaa.Backward(f)
    if dy_bits is not None:
        dyt = torch.from_numpy(dy_bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    else:
        dyt = torch.from_numpy(dy).to(dev)
    outs = []
    for _ in range(repeat):
        f(x["q"], x["k"], x["v"], x["x_gate"], x["hyperplanes"], x["gate_w"], x["gate_b"])
        grads = bwd(x["q"], x["k"], x["v"], x["x_gate"], x["gate_w"], x["gate_b"], dyt)
        torch.cuda.synchronize()
        outs.append([t.float().cpu().numpy().astype(np.float64) for t in grads])
    return outs


@pytest.mark.parametrize("case", list(CASES) + [c + "+saved" for c in SAVED])
def test_backward_parity(case):
    import oracle

    import efficient_long_context_amd as elsaa
    base = case.replace("+saved", "")
    options = elsaa.OPT_SAVE_FOR_BACKWARD if case.endswith("+saved") else 0
    name, over, variant = CASES[base]
    wl = workloads.workload(name, **over)
    inp = workloads.generate(wl, seed=23)
    inp.gate_w *= 20.0  # gates away from one half
    dy, dy_bits = _dy(inp, 29)
    print(f"[backward] {case}: B={wl.B} H={wl.H} N={wl.N} d={wl.d} {wl.dtype} {variant}", flush=True)
    (got,) = run_backward(inp, dy, dy_bits, variant, options=options)
    ref = oracle.backward(inp.q, inp.k, inp.v, inp.x_gate, inp.hyperplanes, inp.gate_w, inp.gate_b, dy,
                          sort_bits=wl.sort_bits, chunk=wl.chunk, race_tables_n=wl.race_tables,
                          race_bits=wl.race_bits, lam=wl.lam, variant=variant)
    names = ("dq", "dk", "dv", "dx_gate", "dgate_w", "dgate_b")
    errs = {n: rel_err(g, getattr(ref, n)) for n, g in zip(names, got[:6])}
    errs["dlambda"] = (abs(got[6][0] - ref.dlambda) / abs(ref.dlambda)) if ref.dlambda != 0 else abs(got[6][0])
    print(f"[backward] {case}: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    tol = TOL[wl.dtype]
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{case}: over tolerance {tol}: {bad}"


def test_backward_deterministic():
    import efficient_long_context_amd as elsaa
    wl = workloads.workload("text32k-bf16", B=1, H=2, N=4096)
    inp = workloads.generate(wl, seed=31)
    dy, dy_bits = _dy(inp, 37)
    for options in (0, elsaa.OPT_SAVE_FOR_BACKWARD):
        a, b = run_backward(inp, dy, dy_bits, "full", repeat=2, options=options)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)
