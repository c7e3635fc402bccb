"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle
on the same seeded inputs.  Codes, permutations and RACE counts must match
bit for bit; floating-point tensors must satisfy max|d| / max|ref| <= 1e-4
(fp32 inputs) or <= 2e-2 (bf16 inputs), per tensor.

Sizes here are ones the oracle finishes in seconds while still spanning many
tiles of every kernel; each workload keeps its own hash settings, chunk,
generator and head dimension, with B, H (and N where needed) reduced.
Full-size runs with per-head properties and oracle-checked slices are in
test_gpu_fullsize.py.
"""
import numpy as np
import pytest

import workloads
from gpu_common import compare_all, compare_variant, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, overrides)
    "tiny-fp32": ("tiny-fp32", {}),
    "small-bf16": ("small-bf16", dict(B=1, H=2)),
    "vision16k-bf16-1head": ("vision16k-bf16", dict(B=1, H=1)),
    "text32k-bf16-1head": ("text32k-bf16", dict(B=1, H=1)),
    "needle-bf16-N16k": ("needle256k-bf16", dict(H=1, N=16384)),
    # edge cases
    "fp32-d128": ("tiny-fp32", dict(d=128, H=2, N=2048, chunk=128)),
    "bf16-ragged-sort-tile": ("small-bf16", dict(B=1, H=3, N=64 * 37, chunk=64)),
    "bf16-single-chunk": ("small-bf16", dict(B=1, H=1, N=64, chunk=64)),
    "bf16-L3-P5": ("small-bf16", dict(B=1, H=2, race_tables=3, race_bits=5)),
    "bf16-P0": ("small-bf16", dict(B=1, H=1, race_bits=0)),
    "bf16-sort12": ("small-bf16", dict(B=1, H=1, N=8192, sort_bits=12)),
    "bf16-P12-L4": ("small-bf16", dict(B=1, H=1, race_tables=4, race_bits=12)),
    "bf16-d128-w64": ("needle256k-bf16", dict(H=2, N=4096, chunk=64, sort_bits=7, race_tables=5, race_bits=9)),
    "bf16-w256": ("small-bf16", dict(B=2, H=2, N=4096, chunk=256)),
    # d = 128 through each bf16 attention kernel: 256-query tiles (w a
    # multiple of 256, two tiles a chunk at w = 512), producer/consumer
    # (w = 128)
    "bf16-d128-w512": ("needle256k-bf16", dict(H=2, N=4096, chunk=512)),
    "bf16-d128-w128": ("needle256k-bf16", dict(H=2, N=4096, chunk=128)),
    # 8-bit codes on byte boundaries: an even number of plane tiles with no
    # sort code, and 12 tables (three code words a row)
    "bf16-bytecodes-ns0-L4": ("small-bf16", dict(B=1, H=2, sort_bits=0, race_tables=4, race_bits=8)),
    "bf16-bytecodes-L12": ("small-bf16", dict(B=1, H=2, race_tables=12, race_bits=8, sort_bits=8)),
    # segments longer than one workgroup's LDS sort: the tiled three-pass sort
    "bf16-long-segment-sort": ("small-bf16", dict(B=1, H=1, N=65536 + 192, chunk=64)),
    # 4096 buckets with 16K codes a segment (the tiled sort: the counters and
    # the codes do not fit one workgroup)
    "bf16-sort12-N16k": ("small-bf16", dict(B=1, H=1, N=16384, sort_bits=12)),
    # the RACE build's tiled rank: 4096 buckets whose counters and 16-bit
    # permutation do not fit one workgroup's LDS (16-bit indices, 4-wave tiles)
    "bf16-race12-N8k": ("small-bf16", dict(B=1, H=2, N=8192, race_tables=2, race_bits=12)),
    # one sort bucket: local-window attention in original order, no sort and no
    # permutation reads, through each attention kernel (sliding-window d = 64
    # w = 128, 256-query tiles d = 128, 64-query tiles, fp32)
    "bf16-ns0-slide": ("text32k-bf16", dict(B=1, H=2, N=4096, sort_bits=0)),
    "bf16-ns0-d128-w256": ("needle256k-bf16", dict(H=2, N=4096, sort_bits=0)),
    "bf16-ns0-w64": ("small-bf16", dict(B=1, H=2, N=2048, sort_bits=0)),
    "fp32-ns0": ("tiny-fp32", dict(sort_bits=0)),
    # no hyperplanes at all (sort_bits = race_bits = 0)
    "bf16-no-planes": ("small-bf16", dict(B=1, H=2, N=2048, sort_bits=0, race_bits=0)),
    "fp32-no-planes": ("tiny-fp32", dict(sort_bits=0, race_bits=0)),
    # gate inputs of other widths: the wide fusion's general gate loop and the
    # any-L fusion with d_gate != 64
    "bf16-dgate48-L16": ("text32k-bf16", dict(B=1, H=2, N=4096, d_gate=48)),
    "bf16-dgate100-L3": ("small-bf16", dict(B=1, H=2, N=2048, race_tables=3, d_gate=100)),
    "fp32-dgate100-L8": ("tiny-fp32", dict(race_tables=8, d_gate=100)),
    # the fusion's LDS path (bfloat16 d = 64, 16 tables, d_gate = 64): 16
    # buckets a table (copies narrower than a wave, counts fewer than 64
    # lanes) with a last tile of 128 queries (six of its eight waves idle),
    # and 2 buckets a table with a last tile of 64 queries
    "bf16-L16-P4-tail": ("text32k-bf16", dict(B=1, H=2, N=4096 + 128, race_bits=4)),
    "bf16-L16-P1-tail": ("text32k-bf16", dict(B=1, H=1, N=2048 + 64, chunk=64, race_bits=1)),
    # the wide fusion at d = 128 with one code byte, and in binary32 with
    # d_gate = 64 (16 and 8 tables)
    "bf16-d128-L16-P8": ("needle256k-bf16", dict(H=2, N=4096, race_bits=8)),
    "fp32-L16": ("tiny-fp32", dict(race_tables=16)),
    "fp32-L8-N2k": ("tiny-fp32", dict(N=2048, race_tables=8, race_bits=6)),
    # the token-blocked RACE build (a (b, h)'s value rows beyond 8 MB): two
    # blocks of 32768 keys at d = 128 with 1024-bucket tables, two blocks of
    # 65536 keys (the 16-bit index limit) at d = 64, four binary32 blocks
    "bf16-race-blocks-d128": ("needle256k-bf16", dict(H=1, N=65536, chunk=64)),
    "bf16-race-blocks-d64": ("text32k-bf16", dict(B=1, H=1, N=131072)),
    "fp32-race-blocks": ("tiny-fp32", dict(N=131072, race_tables=8, race_bits=6)),
    # two blocks of 65536 keys with 2^12-bucket tables: the blocks take the
    # tiled rank (counters and indices beyond one workgroup's LDS), whose tile
    # counts the Sort-LSH tiled sort then reuses
    "bf16-race-blocks-P12": ("small-bf16", dict(B=1, H=1, N=131072, race_tables=4, race_bits=12)),
}


@pytest.mark.parametrize("case", list(CASES))
def test_parity(case):
    name, over = CASES[case]
    wl = workloads.workload(name, **over)
    inp = workloads.generate(wl, seed=11)
    print(f"[parity] {case}: B={wl.B} H={wl.H} N={wl.N} d={wl.d} {wl.dtype}", flush=True)
    g = run_gpu(inp)
    r = run_oracle(inp)
    errs = compare_all(g, r, wl.dtype, case)
    print(f"[parity] {case}: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)


VARIANT_CASES = {
    "tiny-fp32": ("tiny-fp32", {}),
    "text32k-1head": ("text32k-bf16", dict(B=1, H=2, N=4096)),
    "needle-d128": ("needle256k-bf16", dict(H=2, N=4096)),
    "small-L3": ("small-bf16", dict(B=1, H=2, N=2048, race_tables=3, race_bits=5)),
    # a RACE build in two token blocks
    "needle-race-blocks": ("needle256k-bf16", dict(H=1, N=65536, chunk=64)),
}


@pytest.mark.parametrize("variant", ["no_alpha", "race_only", "sparse_only"])
@pytest.mark.parametrize("case", list(VARIANT_CASES))
def test_variant_parity(case, variant):
    """The ablation and the two single-branch models against the oracle's."""
    name, over = VARIANT_CASES[case]
    wl = workloads.workload(name, **over)
    inp = workloads.generate(wl, seed=13)
    print(f"[variant] {case} {variant}: B={wl.B} H={wl.H} N={wl.N} d={wl.d} {wl.dtype}", flush=True)
    g = run_gpu(inp, variant=variant)
    r = run_oracle(inp, variant=variant)
    errs = compare_variant(g, r, wl.dtype, variant, f"{case} {variant}")
    print(f"[variant] {case} {variant}: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)


FUSED_CASES = {
    "text32k-L16": ("text32k-bf16", dict(B=1, H=2, N=4096), "full"),
    "vision16k-L8": ("vision16k-bf16", dict(B=1, H=2), "full"),
    "text32k-ns0": ("text32k-bf16", dict(B=1, H=2, N=4096, sort_bits=0), "full"),
    "text32k-no-alpha": ("text32k-bf16", dict(B=2, H=3, N=2048), "no_alpha"),
    "text32k-lambda0.25": ("text32k-bf16", dict(B=1, H=2, N=2048, lam=0.25), "full"),
}


@pytest.mark.parametrize("case", list(FUSED_CASES))
def test_fused_epilogue_parity(case):
    """The chunk attention with the RACE gather, gates and fusion in its
    epilogue (ELSAA_OPT_FUSED_EPILOGUE) against the oracle."""
    import efficient_long_context_amd as elsaa
    name, over, variant = FUSED_CASES[case]
    wl = workloads.workload(name, **over)
    inp = workloads.generate(wl, seed=19)
    print(f"[fused] {case}: B={wl.B} H={wl.H} N={wl.N}", flush=True)
    g = run_gpu(inp, variant=variant, options=elsaa.OPT_FUSED_EPILOGUE)
    r = run_oracle(inp, variant=variant)
    errs = compare_variant(g, r, wl.dtype, variant, f"fused {case}")
    print(f"[fused] {case}: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)


def test_exact_attention_special_case():
    """sort_bits = 0 and chunk = N: the sparse branch is dense softmax attention."""
    wl = workloads.workload("small-bf16", B=1, H=2, N=1024, chunk=1024, sort_bits=0)
    inp = workloads.generate(wl, seed=5)
    g = run_gpu(inp)
    np.testing.assert_array_equal(g["perm_q"], np.broadcast_to(np.arange(1024), (1, 2, 1024)))
    for h in range(2):
        q = inp.q[0, h].astype(np.float64); k = inp.k[0, h].astype(np.float64)
        v = inp.v[0, h].astype(np.float64)
        s = q @ k.T / np.sqrt(wl.d)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        o = p @ v / p.sum(axis=1, keepdims=True)
        lse = (m[:, 0] + np.log(p.sum(axis=1)))
        assert np.abs(g["o_sparse"][0, h] - o).max() / np.abs(o).max() <= 2e-2
        assert np.abs(g["lse_s"][0, h] - lse).max() / np.abs(lse).max() <= 2e-2


def test_lambda_zero_ablation():
    """lambda = 0 fixes the sparse multiplier to one (the uncorrected hybrid)."""
    wl = workloads.workload("small-bf16", B=1, H=2)
    inp = workloads.generate(wl, seed=6)
    g = run_gpu(inp, lam=0.0)
    assert (g["alpha"] == 1.0).all()
    r = run_oracle(inp, lam=0.0)
    compare_all(g, r, wl.dtype, "lambda0")


@pytest.mark.parametrize("name,over", [
    ("text32k-bf16", dict(B=1, H=2, N=8192)),
    # the token-blocked RACE build: partial tables summed in block order
    ("needle256k-bf16", dict(H=1, N=65536, chunk=64)),
])
def test_deterministic(name, over):
    wl = workloads.workload(name, **over)
    inp = workloads.generate(wl, seed=7)
    a = run_gpu(inp)
    b = run_gpu(inp)
    for key in ("y", "race_sum", "race_cnt", "o_sparse", "lse_s", "perm_q", "perm_k"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


def _integer_inputs(seed, N=2048, H=2, dtype="bf16", scale=1.0, **hash_settings):
    """Small-integer q, k and hyperplanes (times a power of two): many projections are
    exactly zero or tiny, so the exact sign path decides them."""
    settings = dict(race_tables=4, race_bits=5)
    settings.update(hash_settings)
    wl = workloads.workload("small-bf16", B=1, H=H, N=N, dtype=dtype, **settings)
    inp = workloads.generate(wl, seed)
    rng = np.random.default_rng(seed)
    f = (lambda a: a.astype(np.float32))
    sparse = lambda shape: rng.integers(-2, 3, size=shape) * (rng.random(shape) < 0.08)
    q = f(sparse(inp.q.shape) * scale)
    k = f(sparse(inp.k.shape) * scale)
    planes = f(rng.integers(-1, 2, size=inp.hyperplanes.shape))
    if dtype == "bf16":
        to_bits = lambda a: workloads.round_to_bf16_bits(a.astype(np.float64))
        inp.bits["q"], inp.bits["k"], inp.bits["hyperplanes"] = to_bits(q), to_bits(k), to_bits(planes)
    inp.q, inp.k, inp.hyperplanes = q, k, planes
    return inp


@pytest.mark.parametrize("scale,codes", [(1.0, "5-bit"), (2.0 ** 50, "5-bit"), (2.0 ** -50, "5-bit"),
                                          (1.0, "8-bit"), (2.0 ** 50, "8-bit")])
def test_exact_ties_and_extreme_magnitudes(scale, codes):
    """Exact-zero projections (bit 0), rows far outside the certified range
    (|x| > 2^40 or < 2^-40): every such code bit comes from the exact path.
    8-bit codes on byte boundaries take the byte-code output path."""
    hs = {} if codes == "5-bit" else dict(sort_bits=8, race_tables=4, race_bits=8)
    inp = _integer_inputs(21, scale=scale, **hs)
    g = run_gpu(inp)
    r = run_oracle(inp)
    q64 = inp.q.astype(np.float64)
    dots = q64.reshape(-1, q64.shape[-1]) @ inp.hyperplanes.astype(np.float64).T
    assert (dots == 0).mean() > 0.1  # the exact path is exercised
    np.testing.assert_array_equal(g["sort_code_q"], r.sort_code_q)
    np.testing.assert_array_equal(g["sort_code_k"], r.sort_code_k)
    np.testing.assert_array_equal(g["race_code_q"], r.race_code_q)
    np.testing.assert_array_equal(g["race_code_k"], r.race_code_k)
    np.testing.assert_array_equal(g["perm_q"], r.perm_q)
    np.testing.assert_array_equal(g["perm_k"], r.perm_k)


def test_exact_ties_wide_exponent_span():
    """Exact ties whose nonzero products span far more than 39 binary exponents:
    rows are cancelling pairs (c, -c) with c = small integer x 2^e, e in [-30, 30],
    and half of the planes weight both members of each pair equally, so their
    projections are exactly zero with products from 2^-60 to 2^60."""
    wl = workloads.workload("small-bf16", B=1, H=2, N=2048, race_tables=4, race_bits=5)
    inp = workloads.generate(wl, 31)
    rng = np.random.default_rng(31)
    d = wl.d

    def paired(shape):
        c = rng.integers(1, 128, size=shape[:-1] + (d // 2,)) * rng.choice([-1, 1], size=shape[:-1] + (d // 2,))
        c = c * np.exp2(rng.integers(-30, 31, size=c.shape))
        out = np.empty(shape)
        out[..., 0::2], out[..., 1::2] = c, -c
        return out

    q, k = paired(inp.q.shape), paired(inp.k.shape)
    planes = rng.choice([-1.0, 1.0], size=inp.hyperplanes.shape)
    planes[0::2, 1::2] = planes[0::2, 0::2]  # even planes: equal weights within each pair
    to_bits = lambda a: workloads.round_to_bf16_bits(a.astype(np.float64))
    inp.bits["q"], inp.bits["k"], inp.bits["hyperplanes"] = to_bits(q), to_bits(k), to_bits(planes)
    inp.q, inp.k, inp.hyperplanes = q.astype(np.float32), k.astype(np.float32), planes.astype(np.float32)
    dots = inp.q.astype(np.float64).reshape(-1, d) @ planes.T
    assert (dots[:, 0::2] == 0).all() and (dots[:, 1::2] != 0).mean() > 0.99
    g = run_gpu(inp)
    r = run_oracle(inp)
    for key in ("sort_code_q", "sort_code_k", "race_code_q", "race_code_k", "perm_q", "perm_k"):
        np.testing.assert_array_equal(g[key], getattr(r, key), err_msg=key)
