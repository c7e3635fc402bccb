"""Pins for the oracle's backward pass (the exact gradient of its forward pass;
the method's purpose is training: "ELSAA: Efficient Low-Rank and Sparse
Attention Approximation for Training Transformers", first paragraph).

  * Central finite differences of the oracle's forward output, in binary64,
    for every gradient (q, k, v, x_gate, W_g, b_g, lambda) and every variant,
    at coordinates whose perturbation leaves every hash code unchanged (codes
    are piecewise constant and carry no gradient).
  * Closed forms: with one sort bucket and one chunk the sparse-only model is
    dense softmax attention, whose gradient torch's autograd computes on the
    CPU in binary64; with zero RACE bits the RACE-only model averages v, so
    every key's dv is the mean of dy and dq = dk = 0.
"""
import numpy as np
import pytest

import workloads

SETTINGS = dict(sort_bits=2, chunk=16, race_tables_n=3, race_bits=2)


def _inputs(seed=3, **over):
    kw = dict(B=2, H=2, N=64, d=16, sort_bits=2, chunk=16, race_tables=3, race_bits=2, d_gate=8,
              centroids=4)
    kw.update(over)
    wl = workloads.workload("tiny-fp32", **kw)
    inp = workloads.generate(wl, seed)
    inp.gate_w *= 20.0  # gates away from one half, so their gradients are not tiny
    return inp


def _forward(oracle, inp, variant, lam, settings, **repl):
    args = dict(q=inp.q, k=inp.k, v=inp.v, x_gate=inp.x_gate, gate_w=inp.gate_w, gate_b=inp.gate_b)
    args.update(repl)
    return oracle.forward(args["q"], args["k"], args["v"], args["x_gate"], inp.hyperplanes,
                          args["gate_w"], args["gate_b"], lam=lam, variant=variant, **settings)


def _same_codes(a, b):
    return all(np.array_equal(getattr(a, f), getattr(b, f))
               for f in ("perm_q", "perm_k", "race_code_q", "race_code_k"))


@pytest.mark.parametrize("variant", ["full", "no_alpha", "race_only", "sparse_only"])
def test_backward_matches_finite_differences(oracle_lib, variant):
    inp = _inputs()
    rng = np.random.default_rng(1)
    dy = rng.standard_normal(inp.q.shape)
    lam = 0.7
    g = oracle_lib.backward(inp.q, inp.k, inp.v, inp.x_gate, inp.hyperplanes, inp.gate_w, inp.gate_b, dy,
                            lam=lam, variant=variant, **SETTINGS)
    base = _forward(oracle_lib, inp, variant, lam, SETTINGS)
    grads = {"q": g.dq, "k": g.dk, "v": g.dv, "x_gate": g.dx_gate, "gate_w": g.dgate_w, "gate_b": g.dgate_b}
    checked = 0
    for name, grad in grads.items():
        arr = getattr(inp, name).astype(np.float64)
        scale = max(np.abs(grad).max(), 1e-12)
        for _ in range(10):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            h = 1e-5
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += h
            minus[idx] -= h
            rp = _forward(oracle_lib, inp, variant, lam, SETTINGS, **{name: plus})
            rm = _forward(oracle_lib, inp, variant, lam, SETTINGS, **{name: minus})
            if not (_same_codes(rp, base) and _same_codes(rm, base)):
                continue  # a code flips inside the step: no derivative there
            fd = ((rp.y - rm.y) * dy).sum() / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * scale + 1e-9, (name, idx, fd, grad[idx])
            checked += 1
    assert checked >= 40
    rp = _forward(oracle_lib, inp, variant, lam + 1e-6, SETTINGS)
    rm = _forward(oracle_lib, inp, variant, lam - 1e-6, SETTINGS)
    fd = ((rp.y - rm.y) * dy).sum() / 2e-6
    assert abs(fd - g.dlambda) <= 1e-6 * max(abs(fd), 1.0)
    if variant != "full":
        assert g.dlambda == 0.0


def test_backward_lambda_zero_derivative(oracle_lib):
    """At lambda = 0 the multiplier is one, yet its derivative in lambda is
    -Z_lr / Z_s per query: a one-sided difference from lambda = 0 agrees."""
    inp = _inputs(seed=5)
    dy = np.random.default_rng(2).standard_normal(inp.q.shape)
    g = oracle_lib.backward(inp.q, inp.k, inp.v, inp.x_gate, inp.hyperplanes, inp.gate_w, inp.gate_b, dy,
                            lam=0.0, **SETTINGS)
    f = lambda lam: (_forward(oracle_lib, inp, "full", lam, SETTINGS).y * dy).sum()
    h = 1e-6
    fd = (-3 * f(0.0) + 4 * f(h) - f(2 * h)) / (2 * h)  # second-order one-sided
    assert abs(fd - g.dlambda) <= 1e-5 * max(abs(fd), 1.0)
    assert g.dlambda != 0.0


def test_backward_sparse_only_dense_case_matches_autograd(oracle_lib):
    """One sort bucket, one chunk: the sparse-only model is dense softmax
    attention; torch's autograd (CPU, binary64) gives its exact gradient."""
    torch = pytest.importorskip("torch")
    inp = _inputs(seed=7, sort_bits=0, chunk=64)
    dy = np.random.default_rng(3).standard_normal(inp.q.shape)
    settings = dict(SETTINGS, sort_bits=0, chunk=64)
    g = oracle_lib.backward(inp.q, inp.k, inp.v, inp.x_gate, inp.hyperplanes, inp.gate_w, inp.gate_b, dy,
                            lam=1.0, variant="sparse_only", **settings)
    q, k, v = (torch.tensor(a.astype(np.float64), requires_grad=True) for a in (inp.q, inp.k, inp.v))
    s = torch.matmul(q, k.transpose(-1, -2).contiguous()) / np.sqrt(q.shape[-1])
    y = torch.matmul(torch.softmax(s, dim=-1), v)
    (y * torch.tensor(dy)).sum().backward()
    for name, t in (("dq", q), ("dk", k), ("dv", v)):
        np.testing.assert_allclose(getattr(g, name), t.grad.numpy(), rtol=0, atol=1e-12, err_msg=name)


def test_backward_race_only_zero_bits_closed_form(oracle_lib):
    """P = 0: o_lr is the mean of v over all keys, so dv_j = mean_i dy_i for
    every key j, and q and k receive no gradient."""
    inp = _inputs(seed=9, race_bits=0)
    dy = np.random.default_rng(4).standard_normal(inp.q.shape)
    settings = dict(SETTINGS, race_bits=0)
    g = oracle_lib.backward(inp.q, inp.k, inp.v, inp.x_gate, inp.hyperplanes, inp.gate_w, inp.gate_b, dy,
                            lam=1.0, variant="race_only", **settings)
    expect = np.broadcast_to(dy.mean(axis=2, keepdims=True), dy.shape)
    np.testing.assert_allclose(g.dv, expect, rtol=0, atol=1e-13)
    assert not g.dq.any() and not g.dk.any() and not g.dx_gate.any()
