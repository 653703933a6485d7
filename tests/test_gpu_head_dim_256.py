"""Head dim 256 (bf16 inputs only) on the HIP path against the fp64 oracle:
every option of flashbob_bob_ex (causal mask, grouped key/value heads, the
first-backward outputs, a saved log-sum-exp, bf16 outputs), ragged lengths
across several tiles, pass 1 alone, and the fp32 refusal. The sizes stay
small: the oracle's N x N tiles at d = 256 are the slow part here.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_second_order_amd import flashbob as fb
from helpers import NAMES, TOL, make_inputs, rel_fro, say, to_f64

pytestmark = pytest.mark.gpu

D = 256
BF = torch.bfloat16


def device(ins):
    return [ins[k].to("cuda") for k in NAMES]


def check(ins, outs, scale, causal, label, first=False):
    xs = [ins[k].to(torch.float64).numpy() for k in NAMES]
    refs = list(oracle.bob_gqa(*xs, scale, causal=causal))
    if first:
        refs += list(oracle.attention_backward_batched(*xs[:4], scale, causal=causal))
    for k, ref in enumerate(refs):
        e = rel_fro(to_f64(outs[k]), ref)
        assert e <= TOL[BF], f"{label} output {k}: rel {e:.3e}"


@pytest.mark.parametrize("first", [False, True], ids=["bob", "bob+first"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 2)])
def test_d256_options(H, Hkv, causal, first):
    label = f"[d256] H={H} H_kv={Hkv} causal={causal} first={first}"
    say(label)
    ins = make_inputs(1, H, 257, D, BF, seed=2500 + H + 10 * causal + 20 * first, H_kv=Hkv)
    outs = fb.bob(*device(ins), scale=D ** -0.5, causal=causal, first_backward=first)
    torch.cuda.synchronize()
    check(ins, outs, D ** -0.5, causal, label, first)


@pytest.mark.parametrize("N", [1, 2, 33, 130, 300])
def test_d256_ragged(N):
    label = f"[d256] ragged N={N}"
    say(label)
    ins = make_inputs(2, 2, N, D, BF, seed=2600 + N)
    outs = fb.bob(*device(ins), scale=0.07)
    torch.cuda.synchronize()
    xs = [ins[k].to(torch.float64).numpy() for k in NAMES]
    ref = oracle.bob(*xs, 0.07)
    for k in range(4):
        if N == 1 and k < 3:  # exact zeros
            assert np.abs(to_f64(outs[k])).max() <= 1e-5, k
        else:
            assert rel_fro(to_f64(outs[k]), ref[k]) <= TOL[BF], f"{label} output {k}"


def test_d256_saved_lse_and_bf16_outputs():
    say("[d256] saved LSE, bf16 outputs")
    ins = make_inputs(1, 2, 200, D, BF, seed=2700)
    dev = device(ins)
    lse = fb.rowstats(*dev, scale=D ** -0.5)[0]
    got = fb.bob(*dev, scale=D ** -0.5, lse=lse)
    f32 = fb.bob(*dev, scale=D ** -0.5)
    b16 = fb.bob(*dev, scale=D ** -0.5, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    check(ins, got, D ** -0.5, False, "saved LSE")
    for k in range(4):  # bf16 outputs are the float32 results rounded to nearest even
        assert torch.equal(b16[k], f32[k].to(torch.bfloat16)), k


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_d256_rowstats(causal):
    say(f"[d256] rowstats causal={causal}")
    ins = make_inputs(1, 2, 190, D, BF, seed=2800 + causal)
    stats = fb.rowstats(*device(ins), scale=0.05, causal=causal)
    torch.cuda.synchronize()
    for h in range(2):
        xs = [ins[k][0, h].to(torch.float64).numpy() for k in NAMES]
        ref = oracle.row_stats_head(*xs, 0.05, causal=causal)
        for k in range(4):
            got = to_f64(stats[k][0, h])
            assert np.abs(got - ref[k]).max() <= 2e-3 * max(1.0, np.abs(ref[k]).max()), (h, k)


def test_d256_longer():
    label = "[d256] B=1 H=2 N=2048 bf16"
    say(label)
    ins = make_inputs(1, 2, 2048, D, BF, seed=2900)
    outs = fb.bob(*device(ins), scale=D ** -0.5)
    torch.cuda.synchronize()
    xs = [ins[k].to(torch.float64).numpy() for k in NAMES]
    ref = oracle.bob_blocked(*xs, D ** -0.5, block=512)
    for k in range(4):
        assert rel_fro(to_f64(outs[k]), ref[k]) <= TOL[BF], f"{label} output {k}"


def test_d256_float32_refused():
    say("[d256] fp32 refused")
    ins = make_inputs(1, 1, 64, D, torch.float32, seed=3000)
    with pytest.raises(fb.FlashBoBError) as e:
        fb.bob(*device(ins))
    assert e.value.code == -3
