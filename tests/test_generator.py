"""The seeded synthetic workloads: shapes, bfloat16 storage, seed
determinism and the statistics each recipe promises.

Every GPU parity test, the smoke check and the benchmark draw their inputs
from `workloads.generate`; these checks pin the generators themselves to
their recipes (cluster centroids with Gaussian noise; a smooth 2-D Gaussian
random field over a square patch grid; Zipf-distributed token ids over a
32000-word vocabulary; i.i.d. keys with one planted needle key and 16
aligned queries)."""
import numpy as np
import pytest

import workloads

# every workload at a size that generates in well under a second
SMALL = {
    "tiny-fp32": {},
    "small-bf16": dict(B=1, H=2, N=2048),
    "vision16k-bf16": dict(B=1, H=1),          # the 128 x 128 grid is kept whole
    "text32k-bf16": dict(B=1, H=1, N=8192),
    "needle256k-bf16": dict(B=1, H=2, N=4096),
}


def gen(name, seed=0, **over):
    return workloads.generate(workloads.workload(name, **{**SMALL[name], **over}), seed=seed)


@pytest.mark.parametrize("name", list(SMALL))
def test_shapes_and_parameters(name):
    inp = gen(name)
    wl = inp.wl
    assert inp.q.shape == inp.k.shape == inp.v.shape == (wl.B, wl.H, wl.N, wl.d)
    assert inp.x_gate.shape == (wl.B, wl.N, wl.d_gate)
    assert inp.hyperplanes.shape == (wl.sort_bits + wl.race_tables * wl.race_bits, wl.d)
    assert inp.gate_w.shape == (2, wl.H, wl.d_gate) and inp.gate_b.shape == (2, wl.H)
    assert not inp.gate_b.any(), "gate biases start at zero"
    # gate weights N(0, 0.02^2)
    assert abs(inp.gate_w.std() - 0.02) < 0.005
    for x in (inp.q, inp.k, inp.v, inp.x_gate, inp.hyperplanes):
        assert x.dtype == np.float32 and np.isfinite(x).all()


@pytest.mark.parametrize("name", [n for n in SMALL if n.endswith("bf16")])
def test_bf16_storage_is_exact(name):
    inp = gen(name)
    for key in ("q", "k", "v", "x_gate", "hyperplanes"):
        val = getattr(inp, key)
        b = inp.bits[key]
        assert b.dtype == np.uint16 and b.shape == val.shape
        # the stored float32 values are exactly the bf16 patterns
        assert np.array_equal(workloads.bf16_bits_to_f32(b), val)
        # and rounding them again changes nothing (they are representable)
        assert np.array_equal(workloads.round_to_bf16_bits(val.astype(np.float64)), b)


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even
    # significand (1.0); 1 + 3 2^-8 is halfway between 1 + 2^-7 and
    # 1 + 2^-6, whose even neighbour is 1 + 2^-6; just above a tie rounds up
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -30, -(1.0 + 2.0 ** -8), 3.0])
    got = workloads.bf16_bits_to_f32(workloads.round_to_bf16_bits(x)).astype(np.float64)
    np.testing.assert_array_equal(got, [1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -1.0, 3.0])
    # random values: within half an ulp of the 8-bit significand grid
    rng = np.random.default_rng(5)
    y = rng.standard_normal(10000) * 10.0 ** rng.uniform(-3, 3, 10000)
    r = workloads.bf16_bits_to_f32(workloads.round_to_bf16_bits(y)).astype(np.float64)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(y))) - 7)
    assert (np.abs(r - y) <= 0.5 * ulp * (1 + 1e-12)).all()


@pytest.mark.parametrize("name", ["tiny-fp32", "text32k-bf16", "needle256k-bf16"])
def test_seed_determinism(name):
    a, b, c = gen(name, seed=3), gen(name, seed=3), gen(name, seed=4)
    for key in ("q", "k", "v", "x_gate", "hyperplanes", "gate_w"):
        assert np.array_equal(getattr(a, key), getattr(b, key)), key
        assert not np.array_equal(getattr(a, key), getattr(c, key)), key


def test_cluster_recipe():
    # small-bf16: tokens at 128 unit-norm centroids plus N(0, 0.1^2) noise
    inp = gen("small-bf16", H=1, N=4096)
    ids = inp.meta["cluster_ids"][0]
    q = inp.q[0, 0].astype(np.float64)
    assert ids.min() >= 0 and ids.max() < inp.wl.centroids
    means = np.stack([q[ids == c].mean(axis=0) for c in np.unique(ids)])
    # the cluster means sit on the unit sphere (the noise averages out)
    assert np.allclose(np.linalg.norm(means, axis=1), 1.0, atol=0.08)
    resid = q - means[np.searchsorted(np.unique(ids), ids)]
    assert abs(resid.std() - inp.wl.noise) < 0.01
    # queries and keys share the centroid, not the noise
    k = inp.k[0, 0].astype(np.float64)
    assert abs((q - k).std() - np.sqrt(2) * inp.wl.noise) < 0.01


def test_grf_correlation_length():
    # vision16k: a unit-variance Gaussian random field over the 128 x 128
    # patch grid with correlation exp(-r^2 / (2 8^2)), projected to d, plus
    # N(0, 0.2^2) noise
    inp = gen("vision16k-bf16")
    side = 128
    q = inp.q[0, 0].astype(np.float64).reshape(side, side, -1)
    q = q - q.mean(axis=(0, 1))
    var = (q * q).mean()

    def corr(r):  # along the torus rows, averaged over positions and channels
        return (q * np.roll(q, r, axis=0)).mean() / var

    total = 1.0 + inp.wl.noise ** 2  # field variance 1 (per channel, after the projection) + noise
    for r in (1, 4, 8, 16):
        expect = np.exp(-r * r / (2 * 8.0 ** 2)) / total
        assert abs(corr(r) - expect) < 0.08, (r, corr(r), expect)
    assert abs(corr(40)) < 0.05


def test_zipf_token_ids():
    # text32k: token ids Zipf(s = 1.1) over 32000 words; one fixed unit
    # vector per id (per head) plus N(0, 0.1^2) noise
    inp = gen("text32k-bf16", N=32768)
    ids = inp.meta["token_ids"][0]
    assert ids.min() >= 0 and ids.max() < 32000
    counts = np.sort(np.bincount(ids, minlength=32000))[::-1]
    ranks = np.arange(1, 33)
    slope = np.polyfit(np.log(ranks), np.log(counts[:32]), 1)[0]
    assert abs(slope + 1.1) < 0.06, slope
    # rank 1 holds about 1 / H_{32000, 1.1} of the tokens
    h = (np.arange(1, 32001, dtype=np.float64) ** -1.1).sum()
    assert abs(counts[0] / ids.size - 1.0 / h) < 0.02
    # equal ids share one base vector: their queries differ by noise only
    top = np.flatnonzero(ids == np.bincount(ids).argmax())[:64]
    q = inp.q[0, 0][top].astype(np.float64)
    assert abs((q - q.mean(axis=0)).std() - inp.wl.noise) < 0.02
    assert np.allclose(np.linalg.norm(q.mean(axis=0)), 1.0, atol=0.05)


def test_needle_planting():
    # keys and values i.i.d. N(0, 1/d); key at the needle position = 4 q*;
    # 16 aligned queries = q* (exactly, in the stored precision)
    inp = gen("needle256k-bf16")
    d = inp.wl.d
    for h in range(inp.wl.H):
        p = inp.meta["needle_pos"][0, h]
        aligned = inp.meta["aligned_pos"][0, h]
        qstar = inp.meta["qstar"][0, h]
        assert len(set(aligned.tolist())) == 16
        np.testing.assert_array_equal(inp.k[0, h, p].astype(np.float64), 4.0 * qstar)
        for a in aligned:
            np.testing.assert_array_equal(inp.q[0, h, a].astype(np.float64), qstar)
        others = np.delete(inp.k[0, h].astype(np.float64), p, axis=0)
        assert abs(others.var() - 1.0 / d) < 0.05 / d
        assert abs(inp.v[0, h].astype(np.float64).var() - 1.0 / d) < 0.05 / d
