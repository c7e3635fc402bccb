"""The forward pass on two streams at once, and under HIP graph capture.

elsaa_forward runs its sort on a second stream of the device (forked after
the hash, joined before the chunk attention), with the fork and join events
reused under a per-device lock.  Calls from two host threads on two streams
(distinct workspaces, which the header allows to run concurrently) and a
captured graph replayed several times, with eager work and synchronisations
between the replays, must give the eager result bit for bit."""
import threading

import pytest

import workloads
from gpu_common import to_device

pytestmark = pytest.mark.gpu


def _setup(seed):
    import torch

    import efficient_long_context_amd as elsaa
    wl = workloads.workload("text32k-bf16", B=1, H=2, N=4096)
    inp = workloads.generate(wl, seed=seed)
    dev = torch.device("cuda:0")
    x = to_device(inp, dev)
    f = elsaa.Forward(B=wl.B, H=wl.H, N=wl.N, d=wl.d, d_gate=wl.d_gate, sort_bits=wl.sort_bits,
                      chunk=wl.chunk, race_tables=wl.race_tables, race_bits=wl.race_bits, lam=wl.lam,
                      dtype=wl.dtype, device=dev)
    return f, x


def _call(f, x, stream=None):
    return f(x["q"], x["k"], x["v"], x["x_gate"], x["hyperplanes"], x["gate_w"], x["gate_b"], stream=stream)


def test_concurrent_streams_match_serial():
    import torch
    f1, x1 = _setup(21)
    f2, x2 = _setup(22)
    ref1 = _call(f1, x1).clone()
    ref2 = _call(f2, x2).clone()
    torch.cuda.synchronize()
    print("[streams] two threads, two streams, 20 calls each", flush=True)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    errors = []

    def work(f, x, s):
        try:
            for _ in range(20):
                _call(f, x, stream=s)
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(f1, x1, s1)), threading.Thread(target=work, args=(f2, x2, s2))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    assert torch.equal(f1.out, ref1)
    assert torch.equal(f2.out, ref2)


def test_graph_capture_replays_match_eager():
    import torch
    f, x = _setup(23)
    ref = _call(f, x).clone()  # eager (also creates the device's second stream)
    torch.cuda.synchronize()
    print("[graph] capture one forward call, replay three times", flush=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(f, x)
    torch.cuda.synchronize()
    for i in range(3):
        f.out.zero_()
        _call(f, x)  # the program's own eager work between replays
        torch.cuda.synchronize()
        f.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(f.out, ref), f"replay {i}"
