"""Shared helpers of the GPU tests (comparison metrics, device runs, logging)."""

import math
import sys

import numpy as np
import torch

from exact_second_order_amd import flashbob as fb
from exact_second_order_amd.inputs import NAMES, WORKLOADS, make_inputs, workload_inputs  # noqa: F401

# tolerances on the max (over the four outputs) relative Frobenius error
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def say(*a):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(*a, file=sys.stderr, flush=True)


def rel_fro(x, ref, floor=1e-9):
    """||x - ref||_F / ||ref||_F, with the denominator floored at
    floor * sqrt(size): an exact answer of zero (N = 1, zero cotangents) is
    reached by the oracle only up to fp64 rounding, and dividing by that
    rounding residue would not measure anything."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.size == 0:
        return 0.0
    den = max(float(np.linalg.norm(ref)), floor * math.sqrt(ref.size))
    return float(np.linalg.norm(x - ref) / den)


def to_f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def gpu_bob(ins, scale=None, dtype=None, causal=False):
    """Run flashbob.bob on the device; `ins` is the dict of CPU tensors."""
    dev = [ins[k].to("cuda") if dtype is None else ins[k].to(dtype).to("cuda") for k in NAMES]
    out = fb.bob(*dev, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return [o.cpu() for o in out]


def oracle_inputs(ins, b, h):
    return [ins[k][b, h].to(torch.float64).numpy() for k in NAMES]
