"""Capture and concurrency.

The library call inside a captured HIP graph (torch.cuda.CUDAGraph): the C ABI
allocates nothing and records no memset, so a graph of one BoB call with
preallocated outputs and workspace replays to the eager result. It is replayed
several times with eager work and new input values between replays, and every
replay is compared bit for bit with an eager call on the same inputs.

Host threads calling concurrently on their own streams get the results of
serial calls (the library keeps no global state)."""

import pytest
import torch

from exact_second_order_amd import flashbob as fb
from helpers import NAMES, make_inputs, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("causal,first", [(False, False), (True, True)], ids=["plain", "causal+first"])
def test_graph_replay_matches_eager(causal, first):
    say(f"[graph] capture causal={causal} first={first}")
    B, H, N, d = 1, 4, 1000, 64
    ins = make_inputs(B, H, N, d, torch.bfloat16, seed=1800, H_kv=2)
    x = [ins[k].to("cuda") for k in NAMES]
    shapes = fb.shapes_of(B, H, 2, N, d)
    out = [torch.empty(s, dtype=torch.float32, device="cuda") for s in shapes]
    fo = [torch.empty(s, dtype=torch.float32, device="cuda") for s in shapes[:3]] if first else None
    ws = torch.empty(fb.workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream
        fb.bob(*x, out=out, workspace=ws, causal=causal, first_backward=first, first_out=fo)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fb.bob(*x, out=out, workspace=ws, causal=causal, first_backward=first, first_out=fo)
    torch.cuda.synchronize()
    for rep in range(3):
        # new input values in place (the graph holds the pointers)
        new = make_inputs(B, H, N, d, torch.bfloat16, seed=1801 + rep, H_kv=2)
        for t, k in zip(x, NAMES):
            t.copy_(new[k].to("cuda"))
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in out] + ([o.clone() for o in fo] if first else [])
        ref = fb.bob(*x, causal=causal, first_backward=first)
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {rep} output {k} differs from the eager call"


def test_concurrent_host_threads_on_separate_streams():
    # the library keeps no global state: four host threads, each on its own
    # stream with its own problem, get the same results as serial calls
    import threading

    say("[graph] four host threads, four streams")
    probs = [make_inputs(1, 2, 600 + 50 * i, 64, torch.bfloat16, seed=1850 + i) for i in range(4)]
    dev = [[p[k].to("cuda") for k in NAMES] for p in probs]
    ref = [fb.bob(*x, causal=bool(i % 2)) for i, x in enumerate(dev)]
    torch.cuda.synchronize()
    got = [None] * 4
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    got[i] = fb.bob(*dev[i], causal=bool(i % 2), stream=s)
            s.synchronize()
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(4):
        for k in range(4):
            assert torch.equal(got[i][k], ref[i][k]), (i, k)
