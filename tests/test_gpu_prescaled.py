"""Both sides of the pre-scaled dispatch, against the fp64 oracle.

bf16 inputs at d = 64 with |s| = 2^-k (k = 0 .. 59) run pass 1 and pass 2q
with Q and gQ scaled by s in registers (S and G leave the MFMAs scaled,
pass 1 merges r's two sums, pass 2q starts G from -c); every other scale runs
the general kernels. Each case checks the four BoB outputs per head and the
pass-1 row scalars (LSE, D, c, r) per head against the oracle, on a ragged
length spanning several tiles, with and without the causal mask.

Where |s| is large the inputs Q and K are shrunk so that the logits keep the
spread of the default scale (the tolerance is the bf16 parity bar, 2e-2).
"""

import pytest
import torch

import oracle
from exact_second_order_amd import flashbob as fb
from helpers import NAMES, TOL, make_inputs, oracle_inputs, rel_fro, say, to_f64

pytestmark = pytest.mark.gpu

# (scale, factor on Q and K, takes the pre-scaled kernels)
CASES = [
    (1.0, 0.125, True),         # |s| = 2^0, the largest pre-scaled one
    (0.25, 0.5, True),
    (0.125, 1.0, True),          # the default at d = 64
    (-0.125, 1.0, True),         # negative: pass 1 flips the sign, pass 2q scales by s
    (2.0 ** -10, 1.0, True),     # nearly uniform softmax
    (2.0 ** -59, 1.0, True),     # the smallest pre-scaled one
    (2.0 ** -60, 1.0, False),    # just past it: general kernels
    (2.0, 0.0625, False),        # a power of two above 1: general kernels
    (0.13, 1.0, False),
    (-0.3, 0.5, False),
]


def shrunk_inputs(factor, seed, N=300, H=2):
    ins = make_inputs(1, H, N, 64, torch.bfloat16, seed=seed)
    if factor != 1.0:
        for k in ("Q", "K"):
            ins[k] = (ins[k].float() * factor).to(torch.bfloat16)  # a power of two: exact
    return ins


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale,factor,pre", CASES)
def test_bob_both_dispatch_sides(scale, factor, pre, causal):
    label = f"[prescaled] s={scale:g} Q,K x{factor:g} pre={pre} causal={causal}"
    say(label)
    ins = shrunk_inputs(factor, seed=61)
    dev = [ins[k].cuda() for k in NAMES]
    outs = [o.cpu() for o in fb.bob(*dev, scale=scale, causal=causal)]
    torch.cuda.synchronize()
    worst = 0.0
    for h in range(ins["Q"].shape[1]):
        ref = oracle.bob_head(*oracle_inputs(ins, 0, h), scale, causal=causal)
        for k in range(4):
            e = rel_fro(to_f64(outs[k][0, h]), ref[k])
            worst = max(worst, e)
            assert e <= TOL[torch.bfloat16], f"{label} h={h} output {k}: rel {e:.3e}"
    say(f"{label}: worst rel {worst:.3e}")


@pytest.mark.parametrize("scale,factor,pre", CASES)
def test_rowstats_both_dispatch_sides(scale, factor, pre):
    # pass 1 alone (natural row scalars): the pre-scaled finalisation of c and
    # r differs from the general one
    label = f"[prescaled] rowstats s={scale:g} pre={pre}"
    say(label)
    ins = shrunk_inputs(factor, seed=62)
    dev = [ins[k].cuda() for k in NAMES]
    got = [to_f64(t) for t in fb.rowstats(*dev, scale=scale)]
    torch.cuda.synchronize()
    for h in range(ins["Q"].shape[1]):
        ref = oracle.row_stats_head(*oracle_inputs(ins, 0, h), scale)
        for name, g, want in zip(("lse", "D", "c", "r"), got, ref):
            e = rel_fro(g[0, h], want)
            assert e <= 1e-4, f"{label} {name} h={h}: {e:.3e}"
