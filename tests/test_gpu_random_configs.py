"""Randomised configurations of flashbob_bob_ex against the fp64 oracle: each
case draws B, H, H_kv, a ragged N, d, the input dtype, the scale (including
negative values), the mask, the first-backward outputs, a saved LSE and the
output dtype from a seeded generator, so that option combinations no
hand-written test lists are covered too. All outputs are compared; the
generator's seed is in the case name, so a failure names its configuration."""

import numpy as np
import pytest
import torch

import oracle
from exact_second_order_amd import flashbob as fb
from helpers import NAMES, TOL, make_inputs, rel_fro, say, single_key_bounds, to_f64

pytestmark = pytest.mark.gpu

CASES = 40


def draw(seed):
    r = np.random.default_rng(seed)
    Hkv = int(r.choice([1, 2, 3]))
    G = int(r.choice([1, 2, 3]))
    return dict(
        B=int(r.integers(1, 3)), H=Hkv * G, Hkv=Hkv, N=int(r.integers(1, 400)),
        d=int(r.choice([32, 64, 96, 128])),
        dtype=torch.bfloat16 if r.random() < 0.5 else torch.float32,
        scale=float(r.choice([-1.0, 1.0]) * r.uniform(0.05, 0.4)) if r.random() < 0.3 else None,
        causal=bool(r.random() < 0.5), first=bool(r.random() < 0.5), saved=bool(r.random() < 0.3),
        bf16_out=bool(r.random() < 0.3))


@pytest.mark.parametrize("seed", range(CASES))
def test_random_config(seed):
    c = draw(2000 + seed)
    say(f"[random] seed={2000 + seed} {c}")
    ins = make_inputs(c["B"], c["H"], c["N"], c["d"], c["dtype"], seed=3000 + seed, H_kv=c["Hkv"])
    s = c["scale"] if c["scale"] is not None else c["d"] ** -0.5
    xs = [ins[k].to(torch.float64).numpy() for k in NAMES]
    lse = None
    if c["saved"]:
        G = c["H"] // c["Hkv"]
        lse_np = np.empty((c["B"], c["H"], c["N"]))
        for b in range(c["B"]):
            for h in range(c["H"]):
                hx = [xs[i][b, h if k in ("Q", "dO", "gQ") else h // G] for i, k in enumerate(NAMES)]
                lse_np[b, h] = oracle.row_stats_head(*hx, s, causal=c["causal"])[0]
        lse = torch.tensor(lse_np, dtype=torch.float32, device="cuda")
    dev = [ins[k].to("cuda") for k in NAMES]
    outs = fb.bob(*dev, scale=s, causal=c["causal"], first_backward=c["first"], lse=lse,
                  out_dtype=torch.bfloat16 if c["bf16_out"] else torch.float32)
    torch.cuda.synchronize()
    refs = list(oracle.bob_gqa(*xs, s, causal=c["causal"]))
    if c["first"]:
        refs += list(oracle.attention_backward_batched(*xs[:4], s, causal=c["causal"]))
    # bf16 outputs add one rounding (2^-9 relative) to any input dtype
    tol = TOL[c["dtype"]] if not c["bf16_out"] else max(TOL[c["dtype"]], 2e-2)
    assert len(outs) == len(refs)
    for k, (o, ref) in enumerate(zip(outs, refs)):
        got = to_f64(o)
        if np.linalg.norm(ref) < 1e-6 * np.sqrt(ref.size):
            # exact zeros (N = 1): the derived float32 bound, absolute
            # (bf16 outputs round it once more)
            zero = single_key_bounds(ins, s)[0] * (1 + 2.0 ** -8)
            assert np.abs(got).max() <= zero, f"output {k}"
        else:
            e = rel_fro(got, ref)
            assert e <= tol, f"output {k}: rel {e:.3e} > {tol}"


@pytest.mark.parametrize("N,causal", [(64, False), (33, True), (129, False)])
def test_many_short_heads(N, causal):
    # hundreds of heads of a few blocks each (many small workgroups, grouped
    # heads, a single partial block when N < 64)
    B, H, Hkv, d = 8, 16, 4, 64
    say(f"[random] many short heads B={B} H={H} Hkv={Hkv} N={N} causal={causal}")
    ins = make_inputs(B, H, N, d, torch.bfloat16, seed=4000 + N, H_kv=Hkv)
    outs = fb.bob(*[ins[k].to("cuda") for k in NAMES], causal=causal, first_backward=True)
    torch.cuda.synchronize()
    xs = [ins[k].to(torch.float64).numpy() for k in NAMES]
    refs = list(oracle.bob_gqa(*xs, d ** -0.5, causal=causal))
    refs += list(oracle.attention_backward_batched(*xs[:4], d ** -0.5, causal=causal))
    for k, (o, ref) in enumerate(zip(outs, refs)):
        e = rel_fro(to_f64(o), ref)
        assert e <= TOL[torch.bfloat16], f"output {k}: rel {e:.3e}"
