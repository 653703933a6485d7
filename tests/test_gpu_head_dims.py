"""Head dims 32 and 96 (besides 64 and 128) on the HIP path, against the fp64
oracle, with every option of flashbob_bob_ex: both dtypes, with and without
the causal mask, grouped key/value heads, the first-backward outputs and a
saved log-sum-exp; ragged lengths across several tiles, a 4096-length case,
and pass 1 alone.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_second_order_amd import flashbob as fb
from helpers import NAMES, TOL, make_inputs, rel_fro, say, to_f64

pytestmark = pytest.mark.gpu


def device(ins):
    return [ins[k].to("cuda") for k in NAMES]


def check(ins, outs, scale, causal, tol, label, first=False):
    xs = [ins[k].to(torch.float64).numpy() for k in NAMES]
    refs = list(oracle.bob_gqa(*xs, scale, causal=causal))
    if first:
        refs += list(oracle.attention_backward_batched(*xs[:4], scale, causal=causal))
    worst = 0.0
    for k, ref in enumerate(refs):
        e = rel_fro(to_f64(outs[k]), ref)
        worst = max(worst, e)
        assert e <= tol, f"{label} output {k}: rel {e:.3e} > {tol}"
    return worst


@pytest.mark.parametrize("first", [False, True], ids=["bob", "bob+first"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("d", [32, 96])
@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 2)])
def test_head_dim(H, Hkv, d, dtype, causal, first):
    label = f"[dims] B=2 H={H} Hkv={Hkv} N=257 d={d} {dtype} causal={causal} first={first}"
    say(label)
    ins = make_inputs(2, H, 257, d, dtype, seed=1100 + H + Hkv + d, H_kv=Hkv)
    outs = fb.bob(*device(ins), scale=d ** -0.5, causal=causal, first_backward=first)
    torch.cuda.synchronize()
    say(f"{label}: worst rel {check(ins, outs, d ** -0.5, causal, TOL[dtype], label, first):.3e}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("d", [32, 96])
@pytest.mark.parametrize("N", [1, 2, 31, 33, 127, 200, 383, 520])
def test_head_dim_ragged(N, d, dtype):
    label = f"[dims] ragged N={N} d={d} {dtype}"
    say(label)
    ins = make_inputs(1, 2, N, d, dtype, seed=1200 + N + d)
    outs = fb.bob(*device(ins), scale=d ** -0.5)
    torch.cuda.synchronize()
    xs = [ins[k].to(torch.float64).numpy() for k in NAMES]
    ref = oracle.bob(*xs, d ** -0.5)
    for k in range(4):
        if N == 1 and k < 3:  # exact zeros: absolute bound
            assert np.abs(to_f64(outs[k])).max() <= 1e-5, k
        else:
            assert rel_fro(to_f64(outs[k]), ref[k]) <= TOL[dtype], f"{label} output {k}"


@pytest.mark.parametrize("d", [32, 96])
def test_head_dim_saved_lse(d):
    say(f"[dims] saved LSE d={d}")
    ins = make_inputs(1, 2, 300, d, torch.float32, seed=1300 + d)
    dev = device(ins)
    lse = fb.rowstats(*dev, scale=d ** -0.5)[0]
    got = fb.bob(*dev, scale=d ** -0.5, lse=lse)
    torch.cuda.synchronize()
    check(ins, got, d ** -0.5, False, TOL[torch.float32], f"saved d={d}")


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("d", [32, 96])
def test_head_dim_4096_bf16(d, causal):
    label = f"[dims] B=1 H=4 N=4096 d={d} bf16 causal={causal}"
    say(label)
    ins = make_inputs(1, 4, 4096, d, torch.bfloat16, seed=1400 + d)
    outs = fb.bob(*device(ins), scale=d ** -0.5, causal=causal)
    torch.cuda.synchronize()
    xs = [ins[k].to(torch.float64).numpy() for k in NAMES]
    ref = oracle.bob_blocked(*xs, d ** -0.5, block=1024, causal=causal)
    for k in range(4):
        e = rel_fro(to_f64(outs[k]), ref[k])
        assert e <= TOL[torch.bfloat16], f"{label} output {k}: rel {e:.3e}"


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("d", [32, 96])
def test_head_dim_rowstats(d, causal):
    ins = make_inputs(1, 2, 200, d, torch.float32, seed=1500 + d)
    stats = fb.rowstats(*device(ins), scale=0.2, causal=causal)
    torch.cuda.synchronize()
    for h in range(2):
        xs = [ins[k][0, h].to(torch.float64).numpy() for k in NAMES]
        ref = oracle.row_stats_head(*xs, 0.2, causal=causal)
        for k in range(4):
            got = to_f64(stats[k][0, h])
            assert np.abs(got - ref[k]).max() <= 1e-4 * max(1.0, np.abs(ref[k]).max()), (h, k)
