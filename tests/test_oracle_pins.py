"""Pins for the CPU oracle: each oracle stage is checked against something other
than itself -- exact rational arithmetic, correctly rounded summation, numpy's
stable argsort, dense softmax attention, brute-force per-bucket sums, closed
forms and invariants.  None of these checks touches the GPU library.

Sources for the properties pinned (page titles and sections):
  "Two Efficient Attentions, One Denominator Problem": "Two efficient branches can
  still be mis-scaled" (sparse branch exact on the selected pairs; RACE bucket
  summaries; a multiplier on the sparse branch, then independent gates), "The
  ablation isolates the actual contribution" (multiplier fixed to one),
  "Linear interactions are not yet production economics" (interaction count).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import workloads


# ---------------------------------------------------------------- helpers ----

def fsum_sign(x, r):
    """Sign of the exact dot product: products of <=24-bit floats are exact in
    binary64 and math.fsum rounds the exact sum correctly, so the sign is exact."""
    s = math.fsum((float(a) * float(b)) for a, b in zip(x, r))
    return (s > 0) - (s < 0)


def brute_codes(x, planes, first, nbits):
    rows = x.reshape(-1, x.shape[-1])
    out = np.zeros(rows.shape[0], dtype=np.int64)
    for i, row in enumerate(rows):
        c = 0
        for t in range(nbits):
            if fsum_sign(row, planes[first + t]) > 0:
                c += 1 << t
        out[i] = c
    return out.reshape(x.shape[:-1])


def dense_masked_attention(q, k, v, mask):
    """Softmax attention over the keys allowed by mask (binary64, numpy)."""
    d = q.shape[-1]
    s = (q @ k.T) / np.sqrt(d)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    z = p.sum(axis=1, keepdims=True)
    return (p @ v) / z, (m + np.log(z))[:, 0]


def chunk_mask(perm_q, perm_k, w):
    n = perm_q.shape[0]
    rank_q = np.empty(n, dtype=np.int64); rank_q[perm_q] = np.arange(n)
    rank_k = np.empty(n, dtype=np.int64); rank_k[perm_k] = np.arange(n)
    c = rank_q // w
    lo = np.maximum(c - 1, 0) * w
    hi = (c + 1) * w
    return (rank_k[None, :] >= lo[:, None]) & (rank_k[None, :] < hi[:, None])


def small_inputs(dtype="fp32", N=256, d=64, H=2, B=1, sort_bits=4, chunk=32, L=4, P=4, seed=3):
    wl = workloads.workload("tiny-fp32", B=B, H=H, N=N, d=d, dtype=dtype, sort_bits=sort_bits,
                            chunk=chunk, race_tables=L, race_bits=P, centroids=8)
    return workloads.generate(wl, seed)


def run_oracle(oracle, inp, **over):
    wl = inp.wl
    kw = dict(sort_bits=wl.sort_bits, chunk=wl.chunk, race_tables_n=wl.race_tables,
              race_bits=wl.race_bits, lam=wl.lam)
    kw.update(over)
    return oracle.forward(inp.q, inp.k, inp.v, inp.x_gate, inp.hyperplanes, inp.gate_w,
                          inp.gate_b, **kw)


# ------------------------------------------------------------ exact sign ----

def test_exact_sign_matches_rational_arithmetic(oracle_lib):
    rng = np.random.default_rng(0)
    cases = 0
    for trial in range(400):
        d = int(rng.integers(1, 130))
        x = rng.standard_normal(d).astype(np.float32)
        r = rng.standard_normal(d).astype(np.float32)
        if trial % 2 == 0:
            # force heavy cancellation: append exact negatives of earlier products' factors,
            # scaled across wide exponent ranges, plus a tiny residual
            half = d // 2
            x[half:2 * half] = -x[:half]
            r[half:2 * half] = r[:half]
            x[:half] *= np.float32(2.0) ** rng.integers(-40, 40, size=half).astype(np.float32)
            x[half:2 * half] = -x[:half]
            if d % 2 == 1:
                x[-1] = np.float32(rng.choice([0.0, 1e-30, -1e-30, 3e-38]))
        exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x, r))
        want = (exact > 0) - (exact < 0)
        assert oracle_lib.exact_dot_sign(x, r) == want, (trial, d)
        cases += 1
    assert cases == 400


def test_exact_sign_where_naive_binary64_fails(oracle_lib):
    # 1e20 + 1 - 1e20 = 1 exactly; naive left-to-right binary64 gives 0
    x = np.array([1e20, 1.0, -1e20], dtype=np.float32).astype(np.float64)
    assert (x[0] + x[1]) + x[2] == 0.0
    assert oracle_lib.exact_dot_sign(x, np.ones(3)) == 1
    assert oracle_lib.exact_dot_sign(-x, np.ones(3)) == -1
    # exact zero -> sign 0 -> hash bit 0
    z = np.array([2.0 ** -30, 5.0, -5.0, -(2.0 ** -30)])
    assert oracle_lib.exact_dot_sign(z, np.ones(4)) == 0


def test_codes_match_correctly_rounded_sum(oracle_lib):
    inp = small_inputs("bf16", N=128, d=64, H=2, sort_bits=6, L=3, P=5)
    wl = inp.wl
    planes = inp.hyperplanes.astype(np.float64)
    q = inp.q.astype(np.float64)
    got = oracle_lib.srp_codes(q, planes, 0, wl.sort_bits)
    np.testing.assert_array_equal(got, brute_codes(q, planes, 0, wl.sort_bits))
    got_r = oracle_lib.race_codes(q, planes, wl.sort_bits, wl.race_tables, wl.race_bits)
    for l in range(wl.race_tables):
        np.testing.assert_array_equal(
            got_r[..., l], brute_codes(q, planes, wl.sort_bits + l * wl.race_bits, wl.race_bits))


def test_codes_with_exact_ties(oracle_lib):
    # small integers: many dot products are exactly zero and must give bit 0
    rng = np.random.default_rng(1)
    x = rng.integers(-2, 3, size=(300, 8)).astype(np.float64)
    planes = rng.integers(-1, 2, size=(6, 8)).astype(np.float64)
    got = oracle_lib.srp_codes(x, planes, 0, 6)
    want = np.zeros(300, dtype=np.int64)
    dots = x @ planes.T  # exact: small integers
    assert (dots == 0).sum() > 100
    for t in range(6):
        want += (dots[:, t] > 0).astype(np.int64) << t
    np.testing.assert_array_equal(got, want)


def test_code_bit_order_lsb_first(oracle_lib):
    planes = np.eye(4)
    x = np.array([[1.0, -1.0, -1.0, 1.0]])  # planes 0 and 3 positive -> 0b1001
    assert oracle_lib.srp_codes(x, planes, 0, 4)[0] == 0b1001
    assert oracle_lib.srp_codes(x, planes, 1, 3)[0] == 0b100


# -------------------------------------------------------------------- sort ----

def test_stable_sort_matches_numpy_argsort(oracle_lib):
    rng = np.random.default_rng(2)
    for nb, n in [(1, 50), (16, 1000), (1024, 5000), (65536, 3000)]:
        codes = rng.integers(0, nb, size=(3, n)).astype(np.int32)
        got = oracle_lib.stable_sort(codes, nb)
        want = np.argsort(codes, axis=-1, kind="stable")
        np.testing.assert_array_equal(got, want)


# --------------------------------------------------------- sparse branch ----

def test_sparse_branch_single_chunk_is_dense_attention(oracle_lib):
    """sort_bits = 0 and chunk = N: every query attends every key exactly once."""
    inp = small_inputs("fp32", N=512, sort_bits=0, chunk=512)
    r = run_oracle(oracle_lib, inp)
    assert r.pairs == inp.wl.B * inp.wl.H * 512 * 512
    for b in range(inp.wl.B):
        for h in range(inp.wl.H):
            q = inp.q[b, h].astype(np.float64); k = inp.k[b, h].astype(np.float64)
            v = inp.v[b, h].astype(np.float64)
            s = q @ k.T / np.sqrt(q.shape[1])
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            o = p @ v / p.sum(axis=1, keepdims=True)
            lse = np.log(np.exp(s).sum(axis=1))
            np.testing.assert_allclose(r.o_s[b, h], o, rtol=0, atol=1e-12)
            np.testing.assert_allclose(r.lse[b, h], lse, rtol=1e-13, atol=1e-12)
            np.testing.assert_array_equal(r.perm_q[b, h], np.arange(512))


@pytest.mark.parametrize("dtype,chunk,bits", [("fp32", 32, 4), ("bf16", 64, 3), ("fp32", 16, 6)])
def test_sparse_branch_matches_masked_dense(oracle_lib, dtype, chunk, bits):
    inp = small_inputs(dtype, N=256, sort_bits=bits, chunk=chunk)
    r = run_oracle(oracle_lib, inp)
    for b in range(inp.wl.B):
        for h in range(inp.wl.H):
            pq = np.argsort(brute_codes(inp.q[b, h], inp.hyperplanes, 0, bits), kind="stable")
            pk = np.argsort(brute_codes(inp.k[b, h], inp.hyperplanes, 0, bits), kind="stable")
            np.testing.assert_array_equal(r.perm_q[b, h], pq)
            np.testing.assert_array_equal(r.perm_k[b, h], pk)
            mask = chunk_mask(pq, pk, chunk)
            # own chunk + previous chunk: w keys for chunk 0, 2w otherwise
            assert set(mask.sum(axis=1).tolist()) <= {chunk, 2 * chunk}
            o, lse = dense_masked_attention(inp.q[b, h].astype(np.float64),
                                            inp.k[b, h].astype(np.float64),
                                            inp.v[b, h].astype(np.float64), mask)
            np.testing.assert_allclose(r.o_s[b, h], o, rtol=0, atol=1e-12)
            np.testing.assert_allclose(r.lse[b, h], lse, rtol=1e-13, atol=1e-12)


def test_interaction_count_closed_form(oracle_lib):
    inp = small_inputs("fp32", N=512, chunk=64)
    r = run_oracle(oracle_lib, inp)
    N, w = 512, 64
    assert r.pairs == inp.wl.B * inp.wl.H * (N * 2 * w - w * w)


# ----------------------------------------------------------- RACE branch ----

def test_race_tables_brute_force_and_invariants(oracle_lib):
    inp = small_inputs("bf16", N=300, L=5, P=3, chunk=30)
    r = run_oracle(oracle_lib, inp)
    wl = inp.wl
    for b in range(wl.B):
        for h in range(wl.H):
            v = inp.v[b, h].astype(np.float64)
            for l in range(wl.race_tables):
                kc = brute_codes(inp.k[b, h], inp.hyperplanes, wl.sort_bits + l * wl.race_bits,
                                 wl.race_bits)
                np.testing.assert_array_equal(r.race_code_k[b, h, :, l], kc)
                for beta in range(1 << wl.race_bits):
                    sel = kc == beta
                    assert r.race_cnt[b, h, l, beta] == sel.sum()
                    np.testing.assert_allclose(r.race_sum[b, h, l, beta], v[sel].sum(axis=0),
                                               rtol=0, atol=1e-12)
            # invariants: every key lands in exactly one bucket of every table
            np.testing.assert_array_equal(r.race_cnt[b, h].sum(axis=-1), wl.N)
            np.testing.assert_allclose(r.race_sum[b, h].sum(axis=1),
                                       np.broadcast_to(v.sum(axis=0), (wl.race_tables, wl.d)),
                                       rtol=0, atol=1e-10)


def test_race_query_brute_force(oracle_lib):
    inp = small_inputs("fp32", N=200, L=4, P=3, chunk=20)
    r = run_oracle(oracle_lib, inp)
    wl = inp.wl
    for b in range(wl.B):
        for h in range(wl.H):
            v = inp.v[b, h].astype(np.float64)
            qc = r.race_code_q[b, h]; kc = r.race_code_k[b, h]
            # collision matrix summed over tables, then averaged: no tables involved
            coll = sum((qc[:, l][:, None] == kc[:, l][None, :]).astype(np.float64)
                       for l in range(wl.race_tables)) / wl.race_tables
            z = coll.sum(axis=1)
            num = coll @ v
            o = np.where(z[:, None] > 0, num / np.where(z > 0, z, 1.0)[:, None], 0.0)
            np.testing.assert_allclose(r.z_lr[b, h], z, rtol=0, atol=1e-12)
            np.testing.assert_allclose(r.o_lr[b, h], o, rtol=0, atol=1e-12)


def test_race_zero_bits_closed_form(oracle_lib):
    """P = 0: one bucket per table, every query collides with every key."""
    inp = small_inputs("fp32", N=128, L=3, P=0, chunk=32)
    r = run_oracle(oracle_lib, inp)
    np.testing.assert_array_equal(r.z_lr, 128.0)
    mean_v = inp.v.astype(np.float64).mean(axis=2, keepdims=True)
    np.testing.assert_allclose(r.o_lr, np.broadcast_to(mean_v, r.o_lr.shape), rtol=0, atol=1e-12)


def test_race_empty_bucket_gives_zero(oracle_lib):
    sums = np.zeros((1, 2, 4, 3)); counts = np.zeros((1, 2, 4))
    counts[0, :, 1] = 2; sums[0, :, 1] = [1.0, 2.0, 3.0]
    qcodes = np.array([[[1, 1], [0, 0], [1, 0]]], dtype=np.int32)  # [seg, n=3, L=2]
    o, z = oracle_lib.race_query(qcodes, sums, counts, 2)
    np.testing.assert_array_equal(z[0], [2.0, 0.0, 1.0])
    np.testing.assert_allclose(o[0, 0], [0.5, 1.0, 1.5])
    np.testing.assert_array_equal(o[0, 1], [0.0, 0.0, 0.0])
    np.testing.assert_allclose(o[0, 2], [0.5, 1.0, 1.5])  # (1/2)(sum)/(1/2 * 2)


# ------------------------------------------------------ gates and fusion ----

def test_gates_zero_weights_give_one_half(oracle_lib):
    x = np.random.default_rng(4).standard_normal((2, 10, 64))
    g_s, g_lr = oracle_lib.gates(x, np.zeros((2, 3, 64)), np.zeros((2, 3)), 3)
    assert (g_s == 0.5).all() and (g_lr == 0.5).all()


def test_gates_match_logistic(oracle_lib):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 7, 64)); w = rng.standard_normal((2, 3, 64)) * 0.3
    bias = rng.standard_normal((2, 3))
    g_s, g_lr = oracle_lib.gates(x, w, bias, 3)
    for br, g in ((0, g_s), (1, g_lr)):
        a = np.einsum("bnc,hc->bhn", x, w[br]) + bias[br][None, :, None]
        np.testing.assert_allclose(g, 0.5 * (1.0 + np.tanh(a / 2.0)), rtol=1e-14, atol=1e-15)


def test_alpha_is_mass_ratio_and_in_unit_interval(oracle_lib):
    inp = small_inputs("fp32", N=256, chunk=32)
    r = run_oracle(oracle_lib, inp)
    assert (r.alpha >= 0).all() and (r.alpha <= 1).all()
    z_s = np.exp(r.lse)  # small scores: no overflow at this size
    direct = z_s / (z_s + inp.wl.lam * r.z_lr)
    np.testing.assert_allclose(r.alpha, direct, rtol=1e-13, atol=0)
    y = r.g_s[..., None] * r.alpha[..., None] * r.o_s + r.g_lr[..., None] * r.o_lr
    np.testing.assert_allclose(r.y, y, rtol=0, atol=1e-14)


def test_lambda_zero_is_uncorrected_hybrid(oracle_lib):
    """lambda = 0 fixes the sparse multiplier to one: the Sort_Lsh_RACE ablation."""
    inp = small_inputs("fp32", N=256, chunk=32)
    r = run_oracle(oracle_lib, inp, lam=0.0)
    assert (r.alpha == 1.0).all()
    np.testing.assert_allclose(r.y, r.g_s[..., None] * r.o_s + r.g_lr[..., None] * r.o_lr,
                               rtol=0, atol=1e-15)


def test_alpha_large_lse_no_overflow(oracle_lib):
    o = np.ones((3, 2)); lse = np.array([800.0, -800.0, 0.0])
    z = np.array([4.0, 4.0, 0.0]); g = np.full(3, 0.5)
    alpha, y = oracle_lib.fuse(o, lse, o, z, g, g, 1.0)
    assert alpha[0] == 1.0 and 0.0 <= alpha[1] < 1e-300 and alpha[2] == 1.0
    assert np.isfinite(y).all()


# --------------------------------------------------------------- variants ----
# The three relatives of the operator that the pages compare it with ("Two
# Efficient Attentions, One Denominator Problem", sections "The ablation
# isolates the actual contribution" and "Workload structure matters more than
# a single leaderboard"), pinned where they reduce to textbook quantities:
# with one sort bucket and one chunk the sparse branch is dense softmax
# attention, with P = 0 every table has one bucket holding every key, and
# zero gate weights give gates of exactly one half.

def _closed_form_inputs(N=128):
    inp = small_inputs("fp32", N=N, chunk=N, sort_bits=0, P=0, L=3)
    inp.gate_w[...] = 0.0
    inp.gate_b[...] = 0.0
    return inp


def _dense_attention(inp):
    q = inp.q.astype(np.float64); k = inp.k.astype(np.float64); v = inp.v.astype(np.float64)
    s = q @ np.swapaxes(k, -1, -2) / np.sqrt(q.shape[-1])
    m = s.max(axis=-1, keepdims=True)
    p = np.exp(s - m)
    return (p @ v) / p.sum(axis=-1, keepdims=True)


def test_variant_sparse_only_is_dense_attention_at_one_bucket_one_chunk(oracle_lib):
    inp = _closed_form_inputs()
    r = run_oracle(oracle_lib, inp, variant="sparse_only")
    np.testing.assert_allclose(r.y, _dense_attention(inp), rtol=0, atol=1e-12)


def test_variant_race_only_is_mean_value_at_zero_bits(oracle_lib):
    """P = 0: each table's single bucket holds every key, so o_lr is the mean of v."""
    inp = _closed_form_inputs()
    r = run_oracle(oracle_lib, inp, variant="race_only")
    mean_v = inp.v.astype(np.float64).mean(axis=-2, keepdims=True)
    np.testing.assert_allclose(r.y, np.broadcast_to(mean_v, r.y.shape), rtol=0, atol=1e-13)
    np.testing.assert_array_equal(r.z_lr, np.full(r.z_lr.shape, float(inp.wl.N)))


def test_variant_no_alpha_is_half_sum_at_zero_gates(oracle_lib):
    """alpha fixed to one and g = 1/2: y = (dense attention + mean of v) / 2."""
    inp = _closed_form_inputs()
    r = run_oracle(oracle_lib, inp, variant="no_alpha")
    assert (r.alpha == 1.0).all() and (r.g_s == 0.5).all() and (r.g_lr == 0.5).all()
    mean_v = inp.v.astype(np.float64).mean(axis=-2, keepdims=True)
    np.testing.assert_allclose(r.y, 0.5 * (_dense_attention(inp) + mean_v), rtol=0, atol=1e-12)


def test_variant_full_differs_from_no_alpha_only_by_alpha(oracle_lib):
    """With lambda > 0 the full operator's alpha lies strictly inside (0, 1) here,
    and the output is that multiple of the sparse term plus the same low-rank term."""
    inp = _closed_form_inputs()
    full = run_oracle(oracle_lib, inp, variant="full")
    assert ((full.alpha > 0) & (full.alpha < 1)).all()
    mean_v = inp.v.astype(np.float64).mean(axis=-2, keepdims=True)
    y = 0.5 * full.alpha[..., None] * _dense_attention(inp) + 0.5 * mean_v
    np.testing.assert_allclose(full.y, y, rtol=0, atol=1e-12)


def test_unknown_variant_rejected(oracle_lib):
    with pytest.raises(ValueError):
        run_oracle(oracle_lib, _closed_form_inputs(64), variant="bogus")


# -------------------------------------------------------- page-level facts ----

def test_interaction_reduction_matches_pages_order_of_magnitude(oracle_lib):
    """The pages' 32K example: about 1.024e7 attention/bucket interactions against
    1.024e9 dense pairs, roughly 99% fewer (tests/golden/interaction_count.json).
    Counted at the text workload's settings (w=128, L=16) on a 32000-token
    sequence: 2w - w^2/N sparse pairs plus L table lookups per query."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "interaction_count.json")))
    N, w, L = g["N"], 128, 16
    assert N * N == g["dense_pairs"]
    ours = (N - (N % w)) * 2 * w - w * w + L * N  # whole chunks only
    reduction = 1.0 - ours / g["dense_pairs"]
    assert reduction >= g["reduction_at_least"]
    assert ours < 10 * g["elsaa_interactions"]
