"""Seeded synthetic inputs for the ELSAA forward pass.

This module is shared by the tests, the benchmark and the smoke check.  It holds
none of the method's arithmetic (no hashing, sorting, attention, RACE or
fusion): it only draws the inputs -- queries, keys, values, gate inputs,
hyperplanes and gate parameters -- with the shapes and value structure of the
workloads the method is evaluated on, and rounds them to their stored precision.

Workloads (B, H, N, d and hash settings per row of WORKLOADS):
  tiny-fp32      clustered tokens, 32 unit-norm centroids, fp32
  small-bf16     clustered tokens, 128 centroids
  vision16k-bf16 smooth 2-D Gaussian random field over a 128x128 patch grid
                 (correlation length 8 patches) projected per head, plus noise:
                 stands in for the 16K-token image classification tasks
  text32k-bf16   Zipf(1.1) token ids over a 32000-word vocabulary, each id a
                 fixed random unit vector per head, plus noise: stands in for
                 32K-token long-document classification
  needle256k-bf16 i.i.d. keys/values with one planted needle key aligned with
                 16 planted queries: an operator-level needle-in-a-haystack probe
No dataset item is used or reproduced; every value is drawn from a seeded
numpy Generator.

Seeding: numpy.random.SeedSequence(seed).spawn(7) in the fixed order
hyperplanes, gate parameters, q/k structure, q/k noise, v, x_gate, needle.
Values are drawn in binary64 and rounded once, to nearest-even, to the stored
precision.  bf16 tensors are returned as uint16 bit patterns (``*_bits``) and
as their exact float32 values.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "fp32" | "bf16"
    sort_bits: int
    chunk: int
    race_tables: int
    race_bits: int
    lam: float = 1.0
    d_gate: int = 64
    kind: str = "cluster"  # cluster | grf | zipf | needle
    centroids: int = 32
    noise: float = 0.1


WORKLOADS = {
    "tiny-fp32": Workload("tiny-fp32", 1, 1, 1024, 64, "fp32", 4, 64, 4, 4,
                          kind="cluster", centroids=32, noise=0.1),
    "small-bf16": Workload("small-bf16", 4, 8, 4096, 64, "bf16", 6, 64, 8, 6,
                           kind="cluster", centroids=128, noise=0.1),
    "vision16k-bf16": Workload("vision16k-bf16", 8, 8, 16384, 64, "bf16", 8, 128, 8, 8,
                               kind="grf", noise=0.2),
    "text32k-bf16": Workload("text32k-bf16", 2, 12, 32768, 64, "bf16", 8, 128, 16, 8,
                             kind="zipf", noise=0.1),
    "needle256k-bf16": Workload("needle256k-bf16", 1, 8, 262144, 128, "bf16", 10, 256, 16, 10,
                                kind="needle"),
}
ORDER = ["tiny-fp32", "small-bf16", "vision16k-bf16", "text32k-bf16", "needle256k-bf16"]


def workload(name: str, **overrides) -> Workload:
    return replace(WORKLOADS[name], **overrides)


# ----------------------------------------------------------- rounding ----

def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary64 values once, to nearest-even, to bfloat16; return bit patterns.

    Rounding goes straight from binary64 to an 8-significant-bit grid (no
    intermediate float32 rounding, which could round twice).  Subnormal bf16
    values use the fixed 2^-133 grid.  Inputs must be finite and below the
    bf16 overflow threshold.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                  # subnormal range shares one grid
    ulp = np.ldexp(1.0, (e - 8).astype(np.int64))
    r = np.rint(x / ulp) * ulp               # exact scaling; rint is round-half-even
    f = r.astype(np.float32)                 # exact: r has <= 8 significant bits
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Inputs:
    wl: Workload
    q: np.ndarray            # float32 values of the stored tensors (exact)
    k: np.ndarray
    v: np.ndarray
    x_gate: np.ndarray
    hyperplanes: np.ndarray
    gate_w: np.ndarray       # float32 [2, H, d_gate]
    gate_b: np.ndarray       # float32 [2, H]
    bits: dict = field(default_factory=dict)  # bf16 bit patterns, name -> uint16 array
    meta: dict = field(default_factory=dict)  # needle positions etc.


def _store(name: str, x64: np.ndarray, dtype: str, bits: dict) -> np.ndarray:
    if dtype == "fp32":
        return x64.astype(np.float32)
    b = round_to_bf16_bits(x64)
    bits[name] = b
    return bf16_bits_to_f32(b)


def _blur_field(rng, side: int, d: int, corr_len: float) -> np.ndarray:
    """Gaussian random field on a side x side torus, d channels, unit variance.

    White noise blurred by a Gaussian of std corr_len / sqrt(2) (FFT, circular),
    which gives the field a correlation exp(-r^2 / (2 corr_len^2)).
    """
    xi = rng.standard_normal((side, side, d))
    sigma = corr_len / np.sqrt(2.0)
    f = np.fft.fftfreq(side)
    g1 = np.exp(-2.0 * (np.pi * f * sigma) ** 2)  # FT of a unit-mass Gaussian
    kern = g1[:, None] * g1[None, :]
    field_ = np.fft.ifft2(np.fft.fft2(xi, axes=(0, 1)) * kern[:, :, None], axes=(0, 1)).real
    field_ -= field_.mean(axis=(0, 1), keepdims=True)
    field_ /= field_.std(axis=(0, 1), keepdims=True)
    return field_.reshape(side * side, d)


def _zipf_ids(rng, n: int, vocab: int, s: float) -> np.ndarray:
    ranks = np.arange(1, vocab + 1, dtype=np.float64)
    pmf = ranks ** (-s)
    cdf = np.cumsum(pmf)
    cdf /= cdf[-1]
    u = rng.random(n)
    return np.minimum(np.searchsorted(cdf, u, side="right"), vocab - 1)


def generate(wl: Workload | str, seed: int = 0) -> Inputs:
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    ss = np.random.SeedSequence(seed)
    r_planes, r_gate, r_struct, r_noise, r_v, r_x, r_needle = [
        np.random.default_rng(s) for s in ss.spawn(7)]
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    rows = wl.sort_bits + wl.race_tables * wl.race_bits
    bits: dict = {}
    meta: dict = {}

    planes = _store("hyperplanes", r_planes.standard_normal((rows, d)), wl.dtype, bits)
    gate_w = (0.02 * r_gate.standard_normal((2, H, wl.d_gate))).astype(np.float32)
    gate_b = np.zeros((2, H), dtype=np.float32)

    if wl.kind == "cluster":
        mu = r_struct.standard_normal((H, wl.centroids, d))
        mu /= np.linalg.norm(mu, axis=-1, keepdims=True)
        ids = r_struct.integers(0, wl.centroids, size=(B, N))
        base = np.empty((B, H, N, d))
        for h in range(H):
            base[:, h] = mu[h][ids]
        q64 = base + wl.noise * r_noise.standard_normal((B, H, N, d))
        k64 = base + wl.noise * r_noise.standard_normal((B, H, N, d))
        meta["cluster_ids"] = ids
    elif wl.kind == "grf":
        side = int(round(np.sqrt(N)))
        assert side * side == N, "grf workload needs a square patch grid"
        proj = r_struct.standard_normal((H, d, d)) / np.sqrt(d)
        q64 = np.empty((B, H, N, d)); k64 = np.empty((B, H, N, d))
        for b in range(B):
            fld = _blur_field(r_struct, side, d, 8.0)
            for h in range(H):
                base = fld @ proj[h]
                q64[b, h] = base + wl.noise * r_noise.standard_normal((N, d))
                k64[b, h] = base + wl.noise * r_noise.standard_normal((N, d))
    elif wl.kind == "zipf":
        vocab = 32000
        ids = np.stack([_zipf_ids(r_struct, N, vocab, 1.1) for _ in range(B)])
        q64 = np.empty((B, H, N, d)); k64 = np.empty((B, H, N, d))
        for h in range(H):
            emb = r_struct.standard_normal((vocab, d))
            emb /= np.linalg.norm(emb, axis=-1, keepdims=True)
            for b in range(B):
                base = emb[ids[b]]
                q64[b, h] = base + wl.noise * r_noise.standard_normal((N, d))
                k64[b, h] = base + wl.noise * r_noise.standard_normal((N, d))
        meta["token_ids"] = ids
    elif wl.kind == "needle":
        k64 = r_struct.standard_normal((B, H, N, d)) / np.sqrt(d)
        q64 = r_noise.standard_normal((B, H, N, d))
        qstar = r_needle.standard_normal((B, H, d))
        needle_pos = np.empty((B, H), dtype=np.int64)
        aligned = np.empty((B, H, 16), dtype=np.int64)
        for b in range(B):
            for h in range(H):
                p = int(r_needle.integers(0, N))
                needle_pos[b, h] = p
                aligned[b, h] = np.sort(r_needle.choice(N, size=16, replace=False))
        meta["needle_pos"] = needle_pos
        meta["aligned_pos"] = aligned
        # q* is rounded to the stored precision first so that the needle key
        # (4 q*, an exact power-of-two multiple) and the aligned queries carry
        # exactly the stored q*.
        if wl.dtype == "bf16":
            qstar_r = bf16_bits_to_f32(round_to_bf16_bits(qstar)).astype(np.float64)
        else:
            qstar_r = qstar.astype(np.float32).astype(np.float64)
        for b in range(B):
            for h in range(H):
                k64[b, h, needle_pos[b, h]] = 4.0 * qstar_r[b, h]
                q64[b, h, aligned[b, h]] = qstar_r[b, h]
        meta["qstar"] = qstar_r
    else:
        raise ValueError(wl.kind)

    v64 = r_v.standard_normal((B, H, N, d))
    if wl.kind == "needle":
        v64 /= np.sqrt(d)
    x64 = r_x.standard_normal((B, N, wl.d_gate))

    q = _store("q", q64, wl.dtype, bits); del q64
    k = _store("k", k64, wl.dtype, bits); del k64
    v = _store("v", v64, wl.dtype, bits); del v64
    x_gate = _store("x_gate", x64, wl.dtype, bits)
    return Inputs(wl, q, k, v, x_gate, planes, gate_w, gate_b, bits, meta)
