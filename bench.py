"""Benchmark of the ELSAA forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload text32k-bf16]

A step is one whole forward pass (hash, sort, RACE build, chunk attention,
gather/gates/fusion) over one batch of seeded synthetic input already resident
in HBM.  W untimed steps, then K steps timed between two device
synchronisations (no instrumentation inside), then K more steps with the
library's stage events for the per-stage split.  Prints ONE JSON line:
  value        tokens/s (B*N per step) of the whole job
  roofline     the dominant kernel (largest share of the step): algorithmic
               bytes (or flops) per launch over its mean duration, measured with
               HIP events recorded around it on the stream it runs on
  stages       the same figures for every stage
  cpu_baseline the CPU oracle timed on a bounded sample of the same workload on
               this host's cores (whole-job tokens/s extrapolated from the sample)
  parity       GPU vs oracle on the sampled heads
  secondary    the same step timing for the second headline workload
Multi-GPU runs are not supported: every stage is independent per (batch, head),
and this build measures one GPU.
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
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            val = float(row["Counter_Value"]) * 1024.0
            if name.startswith("__amd_rocclr_copyBuffer"):
                calib = max(calib, val)
                continue
            short = name.replace("void ", "").replace("elsaa::(anonymous namespace)::", "").split("(")[0]
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


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="text32k-bf16", choices=list(workloads.WORKLOADS))
    ap.add_argument("--also", default="vision16k-bf16",
                    help="second workload timed the same way ('none' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    def time_workload(name: str, steps: int, warmup: int):
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
        # the timed steps run without stage events; a second pass with the
        # library's stage events (the same number of steps) splits the time
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            f(*call)
        stop.record()
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(stop)
        stage_ev = [ev.create(2 * len(elsaa.STAGES)) for _ in range(steps)]
        for i in range(steps):
            f(*call, stage_events=stage_ev[i])
        torch.cuda.synchronize()
        stage_ms = {st: float(np.mean([ev.elapsed_ms(e[2 * j], e[2 * j + 1]) for e in stage_ev]))
                    for j, st in enumerate(elsaa.STAGES)}
        for e in stage_ev:
            ev.destroy(e)
        out = f.out.float().cpu().numpy()
        return wl, inp, f, total_ms / steps, stage_ms, out, gen_s

    wl, inp, f, ms_step, stage_ms, out, gen_s = time_workload(args.workload, args.steps, args.warmup)
    tokens = wl.B * wl.N
    value = tokens / (ms_step * 1e-3)

    model = stage_model(wl)
    stages = {}
    for st, ms in stage_ms.items():
        m = model[st]
        gbs = m["bytes"] / (ms * 1e-3) / 1e9
        tfl = m["flops"] / (ms * 1e-3) / 1e12
        peak_fl = BF16_PEAK_TFLOPS if m["mfma"] else FP32_PEAK_TFLOPS
        stages[st] = {"ms": round(ms, 5), "alg_bytes": m["bytes"], "alg_flops": m["flops"],
                      "GB_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                      "TFLOP_s": round(tfl, 2), "flop_frac": round(tfl / peak_fl, 4)}
    dom = max(stage_ms, key=stage_ms.get)
    m = model[dom]
    ms = stage_ms[dom]
    # bound: MFMA if the stage's arithmetic intensity exceeds the chip's ridge
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if m["mfma"] and m["flops"] / m["bytes"] > ridge:
        roof = {"bound": "mfma", "achieved": round(m["flops"] / (ms * 1e-3) / 1e12, 2),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(m["bytes"] / (ms * 1e-3) / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(dom, wl.name)
    roof["kernel"] = dom
    roof["ms_per_launch"] = round(ms, 5)

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded generator, no dataset)",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d,
                   "sort_bits": wl.sort_bits, "chunk": wl.chunk, "race_tables": wl.race_tables,
                   "race_bits": wl.race_bits, "lambda": wl.lam, "parallelism": "single GPU"},
        "head_tokens_per_s": round(value * wl.H, 1),
        "roofline": roof,
        "stages": stages,
    }

    if args.also and args.also != "none" and args.also != args.workload:
        wl2, _, _, ms2, st2, _, _ = time_workload(args.also, args.steps, args.warmup)
        result["secondary"] = {"workload": wl2.name, "value": round(wl2.B * wl2.N / (ms2 * 1e-3), 1),
                               "unit": "tokens/s", "ms_per_step": round(ms2, 5),
                               "stages_ms": {k: round(v, 5) for k, v in st2.items()}}

    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        threads = oracle.num_threads()
        heads = args.cpu_heads or 1
        bh_all = [(b, h) for b in range(wl.B) for h in range(wl.H)]
        t_used = 0.0
        done = 0
        errs = []
        exact = True
        for (b, h) in bh_all:
            if done >= heads and (args.cpu_heads or t_used >= 10.0):
                break
            sl = lambda a: np.ascontiguousarray(a[b:b + 1, h:h + 1])
            r = oracle.forward(sl(inp.q), sl(inp.k), sl(inp.v), np.ascontiguousarray(inp.x_gate[b:b + 1]),
                               inp.hyperplanes, np.ascontiguousarray(inp.gate_w[:, h:h + 1]),
                               np.ascontiguousarray(inp.gate_b[:, h:h + 1]), sort_bits=wl.sort_bits,
                               chunk=wl.chunk, race_tables_n=wl.race_tables, race_bits=wl.race_bits,
                               lam=wl.lam)
            t_used += r.seconds
            done += 1
            y = out[b, h]
            errs.append(float(np.abs(y - r.y[0, 0]).max() / np.abs(r.y[0, 0]).max()))
        per_head = t_used / done
        cpu_value = tokens / (per_head * len(bh_all))
        result["cpu_baseline"] = {
            "value": round(cpu_value, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {len(bh_all)} (batch, head) slices of {wl.name} at full N={wl.N}; "
                      f"{t_used:.1f} s of oracle time; whole-job tokens/s extrapolated "
                      f"from the mean time per (batch, head)",
        }
        result["parity"] = {"heads_checked": done, "max_rel_err_y": max(errs),
                            "tolerance": 2e-2 if wl.dtype == "bf16" else 1e-4}

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
