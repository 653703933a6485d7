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


def single_key_bounds(ins, scale):
    """Float32 rounding bounds for rows that see exactly one key (N = 1, or a
    causal first row), where the exact gradQ, gradK, gradV are zero and the
    exact graddO is gV. Returns (bound on |gradQ|, |gradK|, |gradV|, bound on
    |graddO - gV|), both absolute.

    Derivation (u = 2^-24, M = max |input|, s = |scale|, gamma_n = n u / (1 -
    n u), one query i and one key j):
      1. S, dP, H are length-d dot products, the raw G = gQ.K + Q.gK one of
         length 2d; computed in float32 in any order each is off by at most
         gamma times the sum of |terms| (<= d M^2, resp. 2 d M^2; bf16
         products are exact in float32, float32 ones add one rounding, hence
         gamma_{n+1}). Two kernels computing the same product differ by twice
         that.
      2. With one key the row scalars are their one-key values up to a few
         roundings: D = dP, c = G, r = s dP G - D s c + H, so |r - H| <=
         4u s |dP| |G| + 4u |H| (the two product terms are one value rounded
         twice).
      3. P = exp2(s log2(e) S - LSE log2(e)) has argument S2 sl2 -
         round(S1 sl2), so |P - 1| <= 2 s (2 gamma_d + u) d M^2 + 2u =: dp
         (ln 2 log2(e) = 1; exp2 to 2 ulp).
      4. |dS| <= (1 + dp) (2 gamma_d + 4u) d M^2 =: eds,
         |G - c| <= s (2 gamma_2d + 4u) 2 d M^2 =: eg, |A| <= (1 + dp) eg,
         |dS2| <= eds eg + (1 + dp) ((2 gamma_d + 4u) d M^2 + 8u s d^2 M^4).
      5. Each output element is one such term times an input (and one
         rounding): |gradQ|, |gradK| <= (1 + 2u) s (|dS2| + |dS|) M,
         |gradV| <= (1 + 2u) |A| M, |graddO - gV| <= (dp + 2u) M + |A| M.
    """
    u = 2.0 ** -24
    M = float(max(ins[k].float().abs().max() for k in NAMES))
    d = int(ins["Q"].shape[-1])
    s = abs(float(scale))
    f32 = ins["Q"].dtype == torch.float32

    def gamma(n):
        n = n + 1 if f32 else n
        return n * u / (1 - n * u)

    dp = 2 * s * (2 * gamma(d) + u) * d * M * M + 2 * u
    eds = (1 + dp) * (2 * gamma(d) + 4 * u) * d * M * M
    eg = s * (2 * gamma(2 * d) + 4 * u) * 2 * d * M * M
    a = (1 + dp) * eg
    ds2 = eds * eg + (1 + dp) * ((2 * gamma(d) + 4 * u) * d * M * M + 8 * u * s * d * d * M ** 4)
    zero = (1 + 2 * u) * max(s * (ds2 + eds) * M, a * M)
    gdo = (dp + 2 * u) * M + a * M
    return zero, gdo
