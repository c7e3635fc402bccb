"""Benchmark of the ELSAA forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload text32k-bf16]

A step is one whole forward pass (hash, sort, RACE build, chunk attention,
gather/gates/fusion) over one batch of seeded synthetic input already resident
in HBM.  W untimed steps, then K steps timed between two device
synchronisations (no instrumentation inside: ms_per_step and value), then K
steps each bracketed by its own pair of events (median and spread), then K
steps with the library's stage events for the per-stage split.  Prints ONE
JSON line:
  value        tokens/s (B*N per step) of the whole job
  roofline     the dominant kernel (largest share of the step): algorithmic
               bytes (or flops) per launch over its median duration, measured
               with HIP events recorded around it on the stream it runs on
  stages       the same figures for every stage, with % of HBM / MFMA peak and
               % attainable (max(bytes / BW, flops / peak) / t), against the
               published peaks and against the peaks measured on this GPU
  peaks_measured  a 1 GiB device copy (HBM) and a bf16 8192^3 matmul (MFMA)
  backward     the same timing for the backward pass (elsaa_backward)
  cpu_baseline the CPU oracle timed on a bounded sample of the same workload on
               this host's cores (whole-job tokens/s extrapolated from the
               sample), plus a one-thread figure on the small workloads
  parity       GPU vs oracle on the sampled heads
  secondary    the same step timing, roofline, stages, CPU baseline and parity
               for the other headline workloads
Multi-GPU runs are not supported: every stage is independent per (batch, head),
and the benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "ELSAA fwd tokens/sec at N=16K & 32K (1 GPU); % MFMA / % HBM roofline per stage"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
CALIB_BYTES = 256 << 20
KERNEL_FILES = {
    "hash": "k1_hash.hip", "sort": "k2_sort.hip", "race_build": "k4_race_build.hip",
    "chunk_attention": "k3_chunk_attn.hip", "fuse": "k5_fuse.hip",
}


def stage_model(wl: workloads.Workload) -> dict:
    """Algorithmic HBM bytes and flops of each stage for one forward pass.

    Per token-head (s = element bytes, c = RACE code bytes, T = table bytes of
    one (b, h) = L 2^P (d s + 4): bucket sums in the value dtype, counts in
    binary32):
      hash   read 2 d s, write 2 (2 + L c);   flops 2 * 2 d R  (q and k, R planes)
      sort   read 2 * 2 (codes), write 2 * 4 (permutations)
      race   read d s + L c, write T / N
      attn   read 2 * 4 (permutation entries) + 3 d s, write d s + 4;
             flops 4 d per (query, key) pair
      fuse   read L c + T / N + d s + 4 + d_gate s / H, write d s
    """
    s = 2 if wl.dtype == "bf16" else 4
    c = 1 if wl.race_bits <= 8 else 2
    d, L, P, N, H = wl.d, wl.race_tables, wl.race_bits, wl.N, wl.H
    th = wl.B * wl.H * wl.N
    R = wl.sort_bits + L * P
    T = L * (1 << P) * (d * s + 4)
    pairs = wl.B * wl.H * (N * 2 * wl.chunk - wl.chunk * wl.chunk)
    return {
        "hash": dict(bytes=th * (2 * d * s + 2 * (2 + L * c)), flops=th * 2 * 2 * d * R, mfma=wl.dtype == "bf16"),
        "sort": dict(bytes=th * (2 * 2 + 2 * 4), flops=0, mfma=False),
        "race_build": dict(bytes=th * (d * s + L * c) + wl.B * wl.H * T, flops=th * L * (d + 1), mfma=False),
        "chunk_attention": dict(bytes=th * (2 * 4 + 3 * d * s + d * s + 4), flops=4 * d * pairs,
                                mfma=wl.dtype == "bf16"),
        "fuse": dict(bytes=th * (L * c + d * s + 4 + d * s) + wl.B * wl.H * T + wl.B * N * wl.d_gate * s,
                     flops=th * (L * d + 4 * wl.d_gate + 8 * d), mfma=False),
    }


def backward_model(wl: workloads.Workload) -> dict:
    """Algorithmic HBM bytes and MFMA flops of the backward pass, per call.

    Reads q, k, v, dy, o_s (d s each), LSE, the query's and key's L codes and
    the gate inputs once per token-head, the tables once per (b, h); writes
    dq, dk, dv (d s each) and dx_gate.  Flops: the sparse branch's five
    products per (query, key) pair (S, dP, dQ, dK, dV: 2 d each), plus the
    RACE transposes (L d adds per query and per key)."""
    s = 2 if wl.dtype == "bf16" else 4
    c = 1 if wl.race_bits <= 8 else 2
    d, L, P, N = wl.d, wl.race_tables, wl.race_bits, wl.N
    th = wl.B * wl.H * N
    T = L * (1 << P) * (d * s + 4)
    pairs = wl.B * wl.H * (N * 2 * wl.chunk - wl.chunk * wl.chunk)
    rd = th * (5 * d * s + 4 + 2 * L * c) + wl.B * wl.H * T + wl.B * N * wl.d_gate * s
    wr = th * 3 * d * s + wl.B * N * wl.d_gate * s
    return dict(bytes=rd + wr, flops=10 * d * pairs + 2 * th * L * d, mfma=wl.dtype == "bf16")


def source_sha(stage: str) -> str:
    """Hash of the stage's kernel source and the shared kernel header."""
    h = hashlib.sha256()
    for name in (KERNEL_FILES[stage], "elsaa_internal.hpp"):
        h.update(open(os.path.join(ROOT, "efficient_long_context_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(stage: str, workload: str):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE counters, as
    recorded in profiles/traffic.json, or None if absent or taken on a different
    version of the kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[workload][stage]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha") != source_sha(stage):
        return None
    return rec.get("bytes_per_launch")


# Kernel-name prefixes of each stage (a stage's launches, in order).
STAGE_KERNELS = {
    "hash": ("elsaa_k1_hash_",),
    "sort": ("elsaa_k2_sort_",),
    "race_build": ("elsaa_k4_race_",),
    "chunk_attention": ("elsaa_k3_chunk_attn_",),
    "fuse": ("elsaa_k5_fuse",),
}


def record_traffic(workload: str, fetch_csv: str, write_csv: str) -> dict:
    """Turn two rocprofv3 counter runs of this script (--pmc FETCH_SIZE, then
    --pmc WRITE_SIZE, both with --copy-calibration) into HBM bytes per launch
    of each stage, written to profiles/traffic.json.

    The counters read KiB per dispatch.  Each is scaled by what it reads for the
    calibration copy (256 MiB read and 256 MiB written, the largest
    __amd_rocclr_copyBuffer dispatch of the run), so the scale absorbs the
    counter's own units."""
    import csv

    def per_kernel(path, counter):
        sums, counts, calib = {}, {}, 0.0
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        named = []
        for row in rows:
            name = row["Kernel_Name"]
            val = float(row["Counter_Value"]) * 1024.0
            if name.startswith("__amd_rocclr_copyBuffer"):
                calib = max(calib, val)
                continue
            named.append((name.replace("void ", "").replace("elsaa::(anonymous namespace)::", "").split("(")[0], val))
        # A forward call starts at its hash kernel.  The tiled sort's kernels
        # belong to the RACE build's tiled rank when they come before that
        # call's run-table kernel (elsaa_k4_race_runs), which only the tiled
        # rank launches; otherwise they are the Sort-LSH sort's.
        starts = [i for i, (k, _) in enumerate(named) if k.startswith("elsaa_k1_hash_bf16")] + [len(named)]
        tiled_sort = ("elsaa_k2_sort_hist", "elsaa_k2_sort_scan", "elsaa_k2_sort_scatter")
        for c in range(len(starts) - 1):
            call = named[starts[c]:starts[c + 1]]
            runs_at = next((i for i, (k, _) in enumerate(call) if k.startswith("elsaa_k4_race_runs")), -1)
            for i, (short, val) in enumerate(call):
                if short.startswith(tiled_sort) and i < runs_at:
                    short = "elsaa_k4_race_rank_tiles:" + short  # the RACE build's tiled rank
                sums[short] = sums.get(short, 0.0) + val
                counts[short] = counts.get(short, 0) + 1
        if calib <= 0.0:
            raise SystemExit(f"{path}: no calibration copy found (run with --copy-calibration)")
        scale = CALIB_BYTES / calib
        return {k: sums[k] / counts[k] * scale for k in sums}, scale

    fetch, f_scale = per_kernel(fetch_csv, "FETCH_SIZE")
    write, w_scale = per_kernel(write_csv, "WRITE_SIZE")
    rec = {}
    for stage, prefixes in STAGE_KERNELS.items():
        ks = sorted(k for k in fetch if k.startswith(prefixes))
        if not ks:
            continue
        fb = sum(fetch[k] for k in ks)
        wb = sum(write.get(k, 0.0) for k in ks)
        rec[stage] = {"kernels": ks, "fetch_bytes": round(fb), "write_bytes": round(wb),
                      "bytes_per_launch": round(fb + wb), "fetch_scale": round(f_scale, 4),
                      "write_scale": round(w_scale, 4), "source_sha": source_sha(stage)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        allrec = json.load(open(path))
    except (OSError, ValueError):
        allrec = {}
    allrec[workload] = rec
    with open(path, "w") as f:
        json.dump(allrec, f, indent=1, sort_keys=True)
        f.write("\n")
    return rec


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch has loaded."""

    def __init__(self):
        import torch
        self.hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n: int):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            arr[i] = h
        return arr

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def destroy(self, arr):
        for h in arr:
            self.hip.hipEventDestroy(h)


def stage_figures(model: dict, ms: float, peaks: dict) -> dict:
    """Per-stage figures for one stage model entry at `ms` per launch: GB/s and
    TFLOP/s achieved, fractions of the published HBM / MFMA peaks, and the
    fraction of the attainable time max(bytes / BW, flops / peak) against the
    published and the measured peaks."""
    t = ms * 1e-3
    gbs = model["bytes"] / t / 1e9
    tfl = model["flops"] / t / 1e12
    peak_fl = BF16_PEAK_TFLOPS if model["mfma"] else FP32_PEAK_TFLOPS
    attain = max(model["bytes"] / (HBM_PEAK_GBS * 1e9), model["flops"] / (peak_fl * 1e12))
    out = {"ms": round(ms, 5), "alg_bytes": model["bytes"], "alg_flops": model["flops"],
           "GB_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
           "TFLOP_s": round(tfl, 2), "flop_frac": round(tfl / peak_fl, 4),
           "attainable_frac": round(attain / t, 4)}
    if peaks:
        mpk = peaks["mfma_TFLOP_s"] if model["mfma"] else FP32_PEAK_TFLOPS
        attain_m = max(model["bytes"] / (peaks["copy_GB_s"] * 1e9), model["flops"] / (mpk * 1e12))
        out["attainable_frac_measured_peaks"] = round(attain_m / t, 4)
    return out


def measure_peaks(torch, dev) -> dict:
    """Achievable peaks on this GPU: a 1 GiB device-to-device copy (2 GiB of
    HBM traffic per copy) and a bf16 8192 x 8192 x 8192 matmul (hipBLASLt)."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)
    b = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * n * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    e0.record()
    for _ in range(10):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    mfma = 2 * 8192 ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del src, dst, a, b
    torch.cuda.empty_cache()
    return {"copy_GB_s": round(copy_gbs, 1), "mfma_TFLOP_s": round(mfma, 1),
            "copy_frac_of_published": round(copy_gbs / HBM_PEAK_GBS, 4),
            "mfma_frac_of_published": round(mfma / BF16_PEAK_TFLOPS, 4),
            "how": "1 GiB device-to-device copy x10 (2 GiB of traffic each); bf16 8192^3 torch.matmul x10"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the first tens of back-to-back calls after start-up run about 5% slower
    # than the steady state (410 against 430 us a step at text32k); 100 calls
    # take under 50 ms there
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="text32k-bf16", choices=list(workloads.WORKLOADS))
    ap.add_argument("--also", default="vision16k-bf16,needle256k-bf16",
                    help="comma-separated workloads timed the same way ('none' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="(b, h) heads the oracle runs on (0 = enough for ~10 s)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain 256 MiB device copy first (HBM counter calibration)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter CSVs of a run of "
                         "this script into profiles/traffic.json for --workload")
    args = ap.parse_args(argv)

    if args.record_traffic:
        print(json.dumps(record_traffic(args.workload, *args.record_traffic), indent=1))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every ELSAA stage is independent per "
              "(batch, head), so a multi-GPU run would shard heads with no exchange; "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    import efficient_long_context_amd as elsaa

    dev = torch.device("cuda", 0)
    ev = HipEvents()
    if args.copy_calibration:
        # a copy kernel of known size: 256 MiB read + 256 MiB written
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    peaks = {} if args.no_peaks else measure_peaks(torch, dev)

    def event_pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def time_workload(name: str, steps: int, warmup: int, backward: bool):
        wl = workloads.WORKLOADS[name]
        t0 = time.perf_counter()
        inp = workloads.generate(wl, seed=args.seed)
        gen_s = time.perf_counter() - t0
        x = to_device(inp, dev)
        f = elsaa.Forward(B=wl.B, H=wl.H, N=wl.N, d=wl.d, d_gate=wl.d_gate, sort_bits=wl.sort_bits,
                          chunk=wl.chunk, race_tables=wl.race_tables, race_bits=wl.race_bits,
                          lam=wl.lam, dtype=wl.dtype, device=dev)
        call = (x["q"], x["k"], x["v"], x["x_gate"], x["hyperplanes"], x["gate_w"], x["gate_b"])
        for _ in range(warmup):
            f(*call)
        torch.cuda.synchronize()
        # K steps between two synchronisations, no instrumentation inside
        start, stop = event_pair()
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            f(*call)
        stop.record()
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(stop)
        # K steps, each between its own pair of events (median and spread)
        pairs = [event_pair() for _ in range(steps)]
        for a, b in pairs:
            a.record()
            f(*call)
            b.record()
        torch.cuda.synchronize()
        per_step = np.array([a.elapsed_time(b) for a, b in pairs])
        # K steps with the library's stage events (a begin, end pair per stage)
        stage_ev = [ev.create(2 * len(elsaa.STAGES)) for _ in range(steps)]
        for i in range(steps):
            f(*call, stage_events=stage_ev[i])
        torch.cuda.synchronize()
        stage_ms = {st: float(np.median([ev.elapsed_ms(e[2 * j], e[2 * j + 1]) for e in stage_ev]))
                    for j, st in enumerate(elsaa.STAGES)}
        for e in stage_ev:
            ev.destroy(e)
        out = f.out.float().cpu().numpy()
        res = dict(wl=wl, inp=inp, ms_step=total_ms / steps, median_ms=float(np.median(per_step)),
                   p10_ms=float(np.percentile(per_step, 10)), p90_ms=float(np.percentile(per_step, 90)),
                   stage_ms=stage_ms, out=out, gen_s=gen_s)
        if backward:
            # training: the forward keeps what the backward reads (o_lr, counts, gates)
            f = elsaa.Forward(B=wl.B, H=wl.H, N=wl.N, d=wl.d, d_gate=wl.d_gate, sort_bits=wl.sort_bits,
                              chunk=wl.chunk, race_tables=wl.race_tables, race_bits=wl.race_bits,
                              lam=wl.lam, dtype=wl.dtype, options=elsaa.OPT_SAVE_FOR_BACKWARD, device=dev)
            bwd = elsaa.Backward(f)
            rng = np.random.default_rng(args.seed + 1)
            dy = torch.from_numpy(rng.standard_normal((wl.B, wl.H, wl.N, wl.d)).astype(np.float32)).to(dev)
            dy = dy.to(f.tdtype)
            bargs = (x["q"], x["k"], x["v"], x["x_gate"], x["gate_w"], x["gate_b"], dy)
            for _ in range(max(2, warmup // 2)):
                f(*call)
                bwd(*bargs)
            torch.cuda.synchronize()
            bpairs = [event_pair() for _ in range(steps)]
            fpairs = [event_pair() for _ in range(steps)]
            for (a, b), (c, d) in zip(bpairs, fpairs):
                c.record()
                f(*call)  # the backward reads this call's results
                d.record()
                a.record()
                bwd(*bargs)
                b.record()
            torch.cuda.synchronize()
            res["backward_ms"] = float(np.median([a.elapsed_time(b) for a, b in bpairs]))
            res["forward_saving_ms"] = float(np.median([c.elapsed_time(d) for c, d in fpairs]))
        del x, f
        torch.cuda.empty_cache()
        return res

    main_res = time_workload(args.workload, args.steps, args.warmup, backward=not args.no_backward)
    wl, inp, out = main_res["wl"], main_res["inp"], main_res["out"]
    ms_step = main_res["ms_step"]
    tokens = wl.B * wl.N
    value = tokens / (ms_step * 1e-3)

    def roofline(wlx, stage_ms_x):
        """The dominant stage's algorithmic rate against its bound's peak."""
        mx = stage_model(wlx)
        dom = max(stage_ms_x, key=stage_ms_x.get)
        m = mx[dom]
        ms = stage_ms_x[dom]
        # bound: MFMA if the stage's arithmetic intensity exceeds the chip's ridge
        ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        if m["mfma"] and m["flops"] / m["bytes"] > ridge:
            roof = {"bound": "mfma", "achieved": round(m["flops"] / (ms * 1e-3) / 1e12, 2),
                    "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
        else:
            roof = {"bound": "hbm", "achieved": round(m["bytes"] / (ms * 1e-3) / 1e9, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
        roof["traffic"] = measured_traffic(dom, wlx.name)
        roof["kernel"] = dom
        roof["ms_per_launch"] = round(ms, 5)
        roof["timing"] = f"median over {args.steps} launches of the stage's begin/end events"
        return roof

    def cpu_baseline(wlx, inpx, outx):
        """The oracle on (batch, head) slices of the workload at full N, one
        slice at least and then until about 10 s of oracle time (or
        --cpu-heads slices); whole-job tokens/s extrapolated from the mean
        time per slice, and the GPU output's error on those slices."""
        import oracle
        oracle.build(force=False)
        threads = oracle.num_threads()
        heads = args.cpu_heads or 1
        bh_all = [(b, h) for b in range(wlx.B) for h in range(wlx.H)]
        t_used = 0.0
        done = 0
        errs = []
        for (b, h) in bh_all:
            if done >= heads and (args.cpu_heads or t_used >= 10.0):
                break
            sl = lambda a: np.ascontiguousarray(a[b:b + 1, h:h + 1])
            r = oracle.forward(sl(inpx.q), sl(inpx.k), sl(inpx.v), np.ascontiguousarray(inpx.x_gate[b:b + 1]),
                               inpx.hyperplanes, np.ascontiguousarray(inpx.gate_w[:, h:h + 1]),
                               np.ascontiguousarray(inpx.gate_b[:, h:h + 1]), sort_bits=wlx.sort_bits,
                               chunk=wlx.chunk, race_tables_n=wlx.race_tables, race_bits=wlx.race_bits,
                               lam=wlx.lam)
            t_used += r.seconds
            done += 1
            y = outx[b, h]
            errs.append(float(np.abs(y - r.y[0, 0]).max() / np.abs(r.y[0, 0]).max()))
        per_head = t_used / done
        cpu = {
            "value": round(wlx.B * wlx.N / (per_head * len(bh_all)), 2), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} of {len(bh_all)} (batch, head) slices of {wlx.name} at full N={wlx.N}; "
                      f"{t_used:.1f} s of oracle time; whole-job tokens/s extrapolated "
                      f"from the mean time per (batch, head)",
        }
        parity = {"heads_checked": done, "max_rel_err_y": max(errs),
                  "tolerance": 2e-2 if wlx.dtype == "bf16" else 1e-4}
        return cpu, parity

    model = stage_model(wl)
    stage_ms = main_res["stage_ms"]
    stages = {st: stage_figures(model[st], ms, peaks) for st, ms in stage_ms.items()}
    roof = roofline(wl, stage_ms)

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded generator, no dataset)",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d,
                   "sort_bits": wl.sort_bits, "chunk": wl.chunk, "race_tables": wl.race_tables,
                   "race_bits": wl.race_bits, "lambda": wl.lam, "parallelism": "single GPU"},
        "head_tokens_per_s": round(value * wl.H, 1),
        "step_ms": {"median": round(main_res["median_ms"], 5), "p10": round(main_res["p10_ms"], 5),
                    "p90": round(main_res["p90_ms"], 5), "n": args.steps},
        "roofline": roof,
        "stages": stages,
    }
    if peaks:
        result["peaks_measured"] = peaks
    if "backward_ms" in main_res:
        bm = backward_model(wl)
        bms = main_res["backward_ms"]
        result["backward"] = dict(stage_figures(bm, bms, peaks), tokens_per_s=round(tokens / (bms * 1e-3), 1),
                                  forward_with_saving_ms=round(main_res["forward_saving_ms"], 5),
                                  timing=f"median over {args.steps} calls of elsaa_backward, each after a "
                                         f"forward call that saves o_lr, counts and gates for it")

    secondary = []
    for name in (args.also.split(",") if args.also and args.also != "none" else []):
        if name == args.workload:
            continue
        r2 = time_workload(name, args.steps, args.warmup, backward=False)
        wl2 = r2["wl"]
        m2 = stage_model(wl2)
        sec = {"workload": wl2.name, "value": round(wl2.B * wl2.N / (r2["ms_step"] * 1e-3), 1),
               "unit": "tokens/s", "ms_per_step": round(r2["ms_step"], 5),
               "median_ms": round(r2["median_ms"], 5), "roofline": roofline(wl2, r2["stage_ms"]),
               "stages": {st: stage_figures(m2[st], v, peaks) for st, v in r2["stage_ms"].items()}}
        if not args.no_cpu_baseline:
            sec["cpu_baseline"], sec["parity"] = cpu_baseline(wl2, r2["inp"], r2["out"])
        secondary.append(sec)
        del r2
    if secondary:
        result["secondary"] = secondary

    if not args.no_cpu_baseline:
        import oracle
        result["cpu_baseline"], parity = cpu_baseline(wl, inp, out)
        threads = result["cpu_baseline"]["cores"]
        # one thread, whole small workloads
        one = {}
        oracle.set_num_threads(1)
        for name in ("tiny-fp32", "small-bf16"):
            w1 = workloads.WORKLOADS[name]
            i1 = workloads.generate(w1, seed=args.seed)
            r1 = oracle.forward(i1.q, i1.k, i1.v, i1.x_gate, i1.hyperplanes, i1.gate_w, i1.gate_b,
                                sort_bits=w1.sort_bits, chunk=w1.chunk, race_tables_n=w1.race_tables,
                                race_bits=w1.race_bits, lam=w1.lam)
            one[name] = {"seconds": round(r1.seconds, 3),
                         "tokens_per_s": round(w1.B * w1.N / r1.seconds, 1)}
        oracle.set_num_threads(threads)
        result["cpu_baseline"]["one_thread"] = one
        result["parity"] = parity

    print(json.dumps(result))
    return 0


def to_device(inp, device):
    import torch

    def t(name, arr):
        if inp.wl.dtype == "bf16" and name in inp.bits:
            return torch.from_numpy(inp.bits[name].view(np.int16).copy()).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(arr)).to(device)

    return dict(q=t("q", inp.q), k=t("k", inp.k), v=t("v", inp.v), x_gate=t("x_gate", inp.x_gate),
                hyperplanes=t("hyperplanes", inp.hyperplanes),
                gate_w=torch.from_numpy(inp.gate_w).to(device),
                gate_b=torch.from_numpy(inp.gate_b).to(device))


if __name__ == "__main__":
    sys.exit(main())
