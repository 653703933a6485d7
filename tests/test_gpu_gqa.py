"""Parity of grouped key/value heads (GQA / MQA) on the HIP path with the fp64
oracle (oracle.bob_gqa), through the C ABI (flashbob_bob_ex with H_kv < H):
query head h uses key/value head h // (H / H_kv); gradK and gradV sum over
each group. Both dtypes and head dims, ragged lengths, with and without the
causal mask, a 4096-length case, and pass 1 alone.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_second_order_amd import flashbob as fb
from helpers import NAMES, TOL, make_inputs, rel_fro, say, to_f64

pytestmark = pytest.mark.gpu


def run_and_check(B, H, Hkv, N, d, dtype, causal, seed, block=None):
    ins = make_inputs(B, H, N, d, dtype, seed, H_kv=Hkv)
    s = d ** -0.5
    dev = [ins[k].to("cuda") for k in NAMES]
    outs = fb.bob(*dev, scale=s, causal=causal)
    torch.cuda.synchronize()
    assert outs[1].shape == ins["K"].shape and outs[0].shape == ins["Q"].shape
    xs = [ins[k].to(torch.float64).numpy() for k in NAMES]
    ref = oracle.bob_gqa(*xs, s, causal=causal, block=block)
    worst = 0.0
    for k in range(4):
        e = rel_fro(to_f64(outs[k].cpu()), ref[k])
        worst = max(worst, e)
        assert e <= TOL[dtype], f"output {k}: rel {e:.3e}"
    return worst


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,Hkv", [(4, 2), (4, 1), (6, 3)])
def test_gqa_small(H, Hkv, d, dtype, causal):
    say(f"[gqa] H={H} Hkv={Hkv} d={d} {dtype} causal={causal}")
    worst = run_and_check(2, H, Hkv, 257, d, dtype, causal, seed=50 + H + Hkv + d)
    say(f"[gqa] worst rel {worst:.3e}")


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_gqa_4096_bf16(causal):
    say(f"[gqa] B=1 H=8 Hkv=2 N=4096 bf16 causal={causal}")
    worst = run_and_check(1, 8, 2, 4096, 64, torch.bfloat16, causal, seed=77, block=1024)
    say(f"[gqa] worst rel {worst:.3e}")


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_gqa_rowstats(causal):
    ins = make_inputs(1, 4, 200, 64, torch.float32, seed=12, H_kv=2)
    dev = [ins[k].to("cuda") for k in NAMES]
    stats = fb.rowstats(*dev, causal=causal)
    torch.cuda.synchronize()
    for h in range(4):
        xs = [ins[k][0, h if k in ("Q", "dO", "gQ") else h // 2].to(torch.float64).numpy() for k in NAMES]
        ref = oracle.row_stats_head(*xs, 0.125, causal=causal)
        for k in range(4):
            got = to_f64(stats[k][0, h].cpu())
            assert np.abs(got - ref[k]).max() <= 1e-4 * max(1.0, np.abs(ref[k]).max())


def test_gqa_equals_mha_with_repeated_heads():
    # the kernels' group sum against the plain multi-head path on explicitly
    # repeated K, V, gK, gV (both on the device, fp32)
    ins = make_inputs(1, 4, 300, 64, torch.float32, seed=19, H_kv=2)
    dev = {k: ins[k].to("cuda") for k in NAMES}
    g = fb.bob(*[dev[k] for k in NAMES])
    rep = {k: (dev[k].repeat_interleave(2, dim=1).contiguous() if k in ("K", "V", "gK", "gV") else dev[k])
           for k in NAMES}
    m = fb.bob(*[rep[k] for k in NAMES])
    torch.cuda.synchronize()
    for k, (a, b) in enumerate(zip(g, m)):
        if k in (1, 2):
            b = b.view(1, 2, 2, 300, 64).sum(dim=2)
        e = rel_fro(to_f64(a.cpu()), to_f64(b.cpu()))
        assert e <= 1e-5, f"output {k}: {e:.3e}"
