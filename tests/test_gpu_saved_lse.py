"""Pass 1 started from a saved log-sum-exp (flashbob_bob_ex with
FLASHBOB_SAVED_LSE), on the HIP path:

  * with the oracle's LSE: all four outputs against the fp64 oracle, both
    dtypes and head dims, with and without the causal mask and grouped heads,
    ragged lengths; and against the plain call (same values up to rounding);
  * with the LSE that pass 1 itself reports (a forward's saved statistic);
  * with the saved LSE shifted by a constant: the outputs do not change (pass 1
    normalises by the sum it accumulates), which fixes that the saved value
    is used only as a reference point;
  * the 65536-length workload in the benchmark's launch configuration against
    the plain call, and pass 1 alone with the flag through the stage entry.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_second_order_amd import flashbob as fb
from helpers import NAMES, TOL, WORKLOADS, make_inputs, rel_fro, say, to_f64, workload_inputs

pytestmark = pytest.mark.gpu


def oracle_lse(ins, scale, causal):
    """[B, H, N] natural-log LSE of each query row from the fp64 oracle."""
    B, H, N, _ = ins["Q"].shape
    G = H // ins["K"].shape[1]
    out = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            xs = [ins[k][b, h if k in ("Q", "dO", "gQ") else h // G].to(torch.float64).numpy() for k in NAMES]
            out[b, h] = oracle.row_stats_head(*xs, scale, causal=causal)[0]
    return torch.tensor(out, dtype=torch.float32)


def device(ins):
    return [ins[k].to("cuda") for k in NAMES]


# saved-LSE call against the plain call: the row scalars differ by fp32
# rounding only; the bf16 path then rounds P, dS, dS2, A to bf16, where such a
# change flips a few roundings (about 1e-4 relative overall)
SAME = {torch.float32: 1e-5, torch.bfloat16: 1e-3}


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,Hkv,N", [(2, 2, 257), (4, 2, 130)])
def test_saved_lse_vs_oracle(H, Hkv, N, d, dtype, causal):
    label = f"[saved] B=2 H={H} Hkv={Hkv} N={N} d={d} {dtype} causal={causal}"
    say(label)
    s = d ** -0.5
    ins = make_inputs(2, H, N, d, dtype, seed=900 + H + N + d, H_kv=Hkv)
    lse = oracle_lse(ins, s, causal).to("cuda")
    dev = device(ins)
    got = fb.bob(*dev, scale=s, causal=causal, lse=lse)
    plain = fb.bob(*dev, scale=s, causal=causal)
    torch.cuda.synchronize()
    xs = [ins[k].to(torch.float64).numpy() for k in NAMES]
    ref = oracle.bob_gqa(*xs, s, causal=causal)
    for k in range(4):
        e = rel_fro(to_f64(got[k]), ref[k])
        assert e <= TOL[dtype], f"{label} output {k}: rel {e:.3e}"
        e = rel_fro(to_f64(got[k]), to_f64(plain[k]))
        assert e <= SAME[dtype], f"{label} output {k} vs plain call: rel {e:.3e}"


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("N", [1, 2, 33, 200, 383])
def test_saved_lse_ragged_from_pass1(N, causal):
    # the LSE that the library's own pass 1 reports, fed back as a saved one
    say(f"[saved] ragged N={N} causal={causal}")
    ins = make_inputs(1, 2, N, 64, torch.float32, seed=950 + N)
    dev = device(ins)
    lse = fb.rowstats(*dev, scale=0.125, causal=causal)[0]
    got = fb.bob(*dev, scale=0.125, causal=causal, lse=lse)
    plain = fb.bob(*dev, scale=0.125, causal=causal)
    torch.cuda.synchronize()
    for k in range(4):
        # N = 1 has exact zeros in gradQ, gradK, gradV: absolute bound there
        ref = to_f64(plain[k])
        err = np.abs(to_f64(got[k]) - ref).max()
        assert err <= 1e-5 * max(1.0, np.abs(ref).max()), f"output {k}: {err:.3e}"


@pytest.mark.parametrize("shift", [-20.0, -5.0, 5.0, 20.0])
def test_saved_lse_shift_does_not_change_outputs(shift):
    say(f"[saved] shifted LSE {shift}")
    ins = make_inputs(1, 2, 300, 64, torch.float32, seed=31)
    dev = device(ins)
    lse = oracle_lse(ins, 0.125, False).to("cuda") + shift
    got = fb.bob(*dev, scale=0.125, lse=lse)
    plain = fb.bob(*dev, scale=0.125)
    torch.cuda.synchronize()
    for k in range(4):
        e = rel_fro(to_f64(got[k]), to_f64(plain[k]))
        assert e <= 1e-5, f"output {k}: rel {e:.3e}"


def test_saved_lse_negative_scale():
    # pass 1 works with |s| and negated Q, gQ when s < 0; the saved LSE is that
    # of s Q K^T itself
    say("[saved] negative scale")
    ins = make_inputs(1, 2, 200, 64, torch.float32, seed=32)
    dev = device(ins)
    lse = oracle_lse(ins, -0.3, False).to("cuda")
    got = fb.bob(*dev, scale=-0.3, lse=lse)
    torch.cuda.synchronize()
    xs = [ins[k].to(torch.float64).numpy() for k in NAMES]
    ref = oracle.bob(*xs, -0.3)
    for k in range(4):
        assert rel_fro(to_f64(got[k]), ref[k]) <= TOL[torch.float32], k


def test_saved_lse_stage_entry():
    # pass 1 with the saved LSE through the stage entry, then the two pass-2
    # stages without it: same as the plain call
    say("[saved] stage entry")
    ins = make_inputs(1, 2, 300, 64, torch.float32, seed=33)
    dev = device(ins)
    B, H, N, d = 1, 2, 300, 64
    out = [torch.empty(B, H, N, d, dtype=torch.float32, device="cuda") for _ in range(4)]
    ws = torch.empty(fb.workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    lse = fb.rowstats(*dev, scale=0.125)[0]
    fb.bob_stage("pass1", *dev, out, ws, scale=0.125, lse=lse)
    fb.bob_stage("pass2_query", *dev, out, ws, scale=0.125)
    fb.bob_stage("pass2_key", *dev, out, ws, scale=0.125)
    plain = fb.bob(*dev, scale=0.125)
    torch.cuda.synchronize()
    for k in range(4):
        assert rel_fro(to_f64(out[k]), to_f64(plain[k])) <= 1e-5, k


def test_saved_lse_big_workload():
    w = WORKLOADS[3]
    say(f"[saved] {w.name}: saved LSE from pass 1, against the plain call")
    ins = workload_inputs(w)
    dev = device(ins)
    lse = fb.rowstats(*dev, scale=w.scale)[0]
    got = fb.bob(*dev, scale=w.scale, lse=lse)
    plain = fb.bob(*dev, scale=w.scale)
    torch.cuda.synchronize()
    for k in range(4):
        e = rel_fro(to_f64(got[k]), to_f64(plain[k]))
        say(f"[saved] {w.name} output {k}: rel {e:.2e}")
        assert e <= SAME[w.dtype], k


def test_saved_lse_rejects_bad_tensors():
    ins = make_inputs(1, 2, 64, 64, torch.float32, seed=34)
    dev = device(ins)
    with pytest.raises(ValueError):
        fb.bob(*dev, lse=torch.zeros(1, 2, 63, dtype=torch.float32, device="cuda"))
    with pytest.raises(TypeError):
        fb.bob(*dev, lse=torch.zeros(1, 2, 64, dtype=torch.float64, device="cuda"))
