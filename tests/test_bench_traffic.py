"""bench.py's traffic record (host logic, no GPU): counter rows of rocprofv3 are
scaled by the calibration copy and summed per stage, and the tiled sort's
kernels count as the RACE build's tiled rank only before that forward call's
run-table kernel."""
import csv
import json
import os

import bench

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
NS = "void elsaa::(anonymous namespace)::"


def _write(path, counter, kernels):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        # the calibration copy: 256 MiB each way, counted here as 2 x its KiB
        w.writerow({"Dispatch_Id": 0, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter,
                    "Counter_Value": 2 * 256 * 1024})
        for i, (name, kib) in enumerate(kernels, start=1):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": NS + name + "(int)", "Counter_Name": counter,
                        "Counter_Value": kib})


def test_record_traffic_attribution(tmp_path, monkeypatch):
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_sha", lambda stage: "sha-" + stage)
    # call 1: tiled RACE rank (sort kernels, then the run table), gather, then
    # the Sort-LSH sort's own tiled kernels; call 2: the sort beside an LDS
    # rank (its kernels come before the RACE kernels, with no run table)
    call1 = [("elsaa_k1_hash_bf16<128, 11>", 100), ("elsaa_k2_sort_hist<unsigned short, 16>", 10),
             ("elsaa_k2_sort_scan", 2), ("elsaa_k2_sort_scatter<unsigned short, int, 16, false>", 20),
             ("elsaa_k4_race_runs", 1), ("elsaa_k4_race_gather<unsigned short, 128, int>", 400),
             ("elsaa_k2_sort_hist<unsigned short, 4>", 3), ("elsaa_k2_sort_scan", 2),
             ("elsaa_k2_sort_scatter<unsigned short, int, 4, true>", 5)]
    call2 = [("elsaa_k1_hash_bf16<128, 11>", 100), ("elsaa_k2_sort_hist<unsigned short, 4>", 3),
             ("elsaa_k2_sort_scan", 2), ("elsaa_k2_sort_scatter<unsigned short, int, 4, true>", 5),
             ("elsaa_k4_race_rank<unsigned short>", 30), ("elsaa_k4_race_gather<unsigned short, 128, int>", 400)]
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _write(f, "FETCH_SIZE", call1 + call2)
    _write(w, "WRITE_SIZE", call1 + call2)
    rec = bench.record_traffic("x", str(f), str(w))
    kib = 1024.0 / 2  # each counter reads twice the copy's bytes: scale one half
    sort_names = sorted(rec["sort"]["kernels"])
    assert sort_names == ["elsaa_k2_sort_hist<unsigned short, 4>", "elsaa_k2_sort_scan",
                          "elsaa_k2_sort_scatter<unsigned short, int, 4, true>"]
    # the sort's three kernels: (3 + 2 + 5) KiB in both calls (the plain scan
    # of call 1 averages with its own tiled-rank twin under another name)
    assert rec["sort"]["fetch_bytes"] == round((3 + 2 + 5) * kib)
    race = rec["race_build"]
    assert "elsaa_k4_race_rank_tiles:elsaa_k2_sort_hist<unsigned short, 16>" in race["kernels"]
    assert "elsaa_k4_race_rank_tiles:elsaa_k2_sort_scan" in race["kernels"]
    # per-launch means over the calls that ran each kernel
    assert race["fetch_bytes"] == round((10 + 2 + 20 + 1 + 400 + 30) * kib)
    assert rec["hash"]["fetch_bytes"] == round(100 * kib)
    assert rec["race_build"]["source_sha"] == "sha-race_build"
    assert json.load(open(tmp_path / "profiles" / "traffic.json"))["x"]["sort"]["kernels"] == rec["sort"]["kernels"]
