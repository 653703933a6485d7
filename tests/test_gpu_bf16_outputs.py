"""bf16 outputs (flashbob_bob_ex with FLASHBOB_BF16_OUTPUTS): the same kernels
store their float32 results rounded to nearest even, so every output must equal,
bit for bit, the float32-output call's result rounded by torch. Checked for
every head dim, both input dtypes, the mask, grouped heads, the first backward,
a saved LSE, the stage entry, and the 65536-length workload in the benchmark's
launch configuration (whose bf16 outputs are also checked against the oracle
on sampled rows).
"""

import numpy as np
import pytest
import torch

import oracle
from exact_second_order_amd import flashbob as fb
from helpers import NAMES, TOL, WORKLOADS, make_inputs, rel_fro, say, to_f64, workload_inputs

pytestmark = pytest.mark.gpu


def device(ins):
    return [ins[k].to("cuda") for k in NAMES]


def assert_rounded(got_bf16, ref_f32, label):
    for k, (g, r) in enumerate(zip(got_bf16, ref_f32)):
        assert g.dtype == torch.bfloat16 and g.shape == r.shape
        want = r.to(torch.bfloat16)
        same = torch.equal(g.view(torch.int16), want.view(torch.int16))
        if not same:
            n = int((g.view(torch.int16) != want.view(torch.int16)).sum())
            raise AssertionError(f"{label} output {k}: {n} of {g.numel()} elements differ from RNE(float32)")


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 96, 128])
def test_bf16_outputs_match_rounded_f32(d, dtype, causal):
    label = f"[bf16out] B=2 H=4 Hkv=2 N=300 d={d} {dtype} causal={causal}"
    say(label)
    ins = make_inputs(2, 4, 300, d, dtype, seed=1600 + d, H_kv=2)
    dev = device(ins)
    for first in (False, True):
        ref = fb.bob(*dev, causal=causal, first_backward=first)
        got = fb.bob(*dev, causal=causal, first_backward=first, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert_rounded(got, ref, f"{label} first={first}")


def test_bf16_outputs_saved_lse_and_stages():
    say("[bf16out] saved LSE, stage entry")
    ins = make_inputs(1, 2, 200, 64, torch.bfloat16, seed=1700)
    dev = device(ins)
    lse = fb.rowstats(*dev)[0]
    ref = fb.bob(*dev, lse=lse)
    got = fb.bob(*dev, lse=lse, out_dtype=torch.bfloat16)
    out = [torch.empty(1, 2, 200, 64, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    ws = torch.empty(fb.workspace_bytes(1, 2, 200, 64), dtype=torch.uint8, device="cuda")
    for st in fb.STAGES:
        fb.bob_stage(st, *dev, out, ws)
    plain = fb.bob(*dev)
    torch.cuda.synchronize()
    assert_rounded(got, ref, "saved LSE")
    assert_rounded(out, plain, "stage entry")


def test_bf16_outputs_mixed_tensors_rejected():
    ins = make_inputs(1, 2, 64, 64, torch.bfloat16, seed=1701)
    dev = device(ins)
    out = [torch.empty(1, 2, 64, 64, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    out.append(torch.empty(1, 2, 64, 64, dtype=torch.float32, device="cuda"))
    ws = torch.empty(fb.workspace_bytes(1, 2, 64, 64), dtype=torch.uint8, device="cuda")
    with pytest.raises(TypeError):
        fb.bob_stage("pass2_query", *dev, out, ws)
    with pytest.raises(TypeError):
        fb.bob(*dev, out_dtype=torch.float16)


def test_bf16_outputs_big_workload():
    w = WORKLOADS[3]
    say(f"[bf16out] {w.name}")
    ins = workload_inputs(w)
    dev = device(ins)
    ref = fb.bob(*dev, scale=w.scale)
    got = fb.bob(*dev, scale=w.scale, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_rounded(got, ref, w.name)
    # and against the oracle on a sampled block of rows (gradQ, graddO)
    rows = np.arange(4096, 4096 + 128)
    for h in range(w.H):
        xs = [ins[k][0, h].to(torch.float64).numpy() for k in NAMES]
        gq, gdo = oracle.bob_rows_head(*xs, w.scale, rows)
        assert rel_fro(to_f64(got[0][0, h][rows]), gq) <= TOL[torch.bfloat16]
        assert rel_fro(to_f64(got[3][0, h][rows]), gdo) <= TOL[torch.bfloat16]
