"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
library through its C ABI with every per-stage output requested, run the
oracle on the same inputs, and compare."""
from __future__ import annotations

import numpy as np

import workloads

TOL = {"bf16": 2e-2, "fp32": 1e-4}


def to_device(inp: workloads.Inputs, device):
    import torch

    def t(name, arr):
        if inp.wl.dtype == "bf16" and name in inp.bits:
            return torch.from_numpy(inp.bits[name].view(np.int16).copy()).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(arr)).to(device)

    return dict(q=t("q", inp.q), k=t("k", inp.k), v=t("v", inp.v), x_gate=t("x_gate", inp.x_gate),
                hyperplanes=t("hyperplanes", inp.hyperplanes),
                gate_w=torch.from_numpy(inp.gate_w).to(device),
                gate_b=torch.from_numpy(inp.gate_b).to(device))


def run_gpu(inp: workloads.Inputs, lam=None, device="cuda:0", variant="full", options=0):
    import torch

    import efficient_long_context_amd as elsaa
    wl = inp.wl
    dev = torch.device(device)
    x = to_device(inp, dev)
    f = elsaa.Forward(B=wl.B, H=wl.H, N=wl.N, d=wl.d, d_gate=wl.d_gate, sort_bits=wl.sort_bits,
                      chunk=wl.chunk, race_tables=wl.race_tables, race_bits=wl.race_bits,
                      lam=wl.lam if lam is None else lam, dtype=wl.dtype, variant=variant,
                      options=options, device=dev, aux=True)
    out = f(x["q"], x["k"], x["v"], x["x_gate"], x["hyperplanes"], x["gate_w"], x["gate_b"])
    torch.cuda.synchronize()
    res = {"y": out.float().cpu().numpy().astype(np.float64)}
    for name, tensor in f.aux.items():
        a = tensor.cpu()
        if name in ("sort_code_q", "sort_code_k"):
            a = a.numpy().view(np.uint16).astype(np.int64)
        elif name in ("race_code_q", "race_code_k"):
            a = a.numpy()
            a = (a.view(np.uint16) if a.dtype == np.int16 else a).astype(np.int64)
        elif tensor.dtype in (torch.int32, torch.int64):
            a = a.numpy()
        else:
            a = a.float().numpy().astype(np.float64)
        res[name] = a
    return res


def run_oracle(inp: workloads.Inputs, lam=None, variant="full"):
    import oracle
    wl = inp.wl
    return oracle.forward(inp.q, inp.k, inp.v, inp.x_gate, inp.hyperplanes, inp.gate_w,
                          inp.gate_b, sort_bits=wl.sort_bits, chunk=wl.chunk,
                          race_tables_n=wl.race_tables, race_bits=wl.race_bits,
                          lam=wl.lam if lam is None else lam, variant=variant)


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.abs(ref).max()
    if denom == 0.0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / denom)


def compare_all(g: dict, r, dtype: str, label: str = "") -> dict:
    """Bit-exact codes, permutations and counts; tolerance on floating outputs."""
    tol = TOL[dtype]
    np.testing.assert_array_equal(g["sort_code_q"], r.sort_code_q, err_msg=label + " sort_code_q")
    np.testing.assert_array_equal(g["sort_code_k"], r.sort_code_k, err_msg=label + " sort_code_k")
    np.testing.assert_array_equal(g["race_code_q"], r.race_code_q, err_msg=label + " race_code_q")
    np.testing.assert_array_equal(g["race_code_k"], r.race_code_k, err_msg=label + " race_code_k")
    np.testing.assert_array_equal(g["perm_q"], r.perm_q, err_msg=label + " perm_q")
    np.testing.assert_array_equal(g["perm_k"], r.perm_k, err_msg=label + " perm_k")
    np.testing.assert_array_equal(g["race_cnt"], r.race_cnt, err_msg=label + " race_cnt")
    errs = {
        "race_sum": rel_err(g["race_sum"], r.race_sum),
        "o_sparse": rel_err(g["o_sparse"], r.o_s),
        "lse_s": rel_err(g["lse_s"], r.lse),
        "z_lr": rel_err(g["z_lr"], r.z_lr),
        "o_lowrank": rel_err(g["o_lowrank"], r.o_lr),
        "g_s": rel_err(g["g_s"], r.g_s),
        "g_lr": rel_err(g["g_lr"], r.g_lr),
        "alpha": rel_err(g["alpha"], r.alpha),
        "y": rel_err(g["y"], r.y),
    }
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{label}: over tolerance {tol}: {bad}"
    assert (g["alpha"] >= 0).all() and (g["alpha"] <= 1).all()
    return errs


def compare_variant(g: dict, r, dtype: str, variant: str, label: str = "") -> dict:
    """As compare_all, restricted to the outputs the variant produces: the
    branch-only variants leave the skipped branch's per-stage outputs
    unwritten."""
    if variant in ("full", "no_alpha"):
        errs = compare_all(g, r, dtype, label)
        if variant == "no_alpha":
            assert (g["alpha"] == 1.0).all(), label + " alpha"
        return errs
    tol = TOL[dtype]
    if variant == "race_only":
        exact = ("race_code_q", "race_code_k", "race_cnt")
        close = {"race_sum": r.race_sum, "z_lr": r.z_lr, "o_lowrank": r.o_lr, "y": r.y}
    else:
        exact = ("sort_code_q", "sort_code_k", "perm_q", "perm_k")
        close = {"o_sparse": r.o_s, "lse_s": r.lse, "y": r.y}
    for key in exact:
        np.testing.assert_array_equal(g[key], getattr(r, key), err_msg=f"{label} {key}")
    errs = {key: rel_err(g[key], ref) for key, ref in close.items()}
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{label}: over tolerance {tol}: {bad}"
    return errs
