"""Parity of the causal HIP BoB path (query i attends to keys j <= i) with the
causal fp64 oracle, through the C ABI (flashbob_bob_ex / flashbob_rowstats_ex
with FLASHBOB_CAUSAL).

  * the 128- and 4096-length workloads: full oracle, every output element;
  * ragged lengths across the diagonal tiles, both head dims and dtypes;
  * the 65536-length workload in the benchmark's launch configuration:
    oracle rows for the first, the last and a sampled block of 256 queries
    per head, fp32-vs-bf16 consistency, and key-shift invariance (which the
    mask keeps: the shift is constant over each row's visible keys);
  * the first query row, fixed in closed form (gradQ = 0, graddO = gV);
  * pass 1 alone against the oracle's causal row scalars.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_second_order_amd import flashbob as fb
from helpers import (NAMES, TOL, WORKLOADS, gpu_bob, make_inputs, oracle_inputs, rel_fro, say,
                     single_key_bounds, to_f64, workload_inputs)

pytestmark = pytest.mark.gpu


def check_heads(ins, outs, scale, tol, label):
    B, H = ins["Q"].shape[:2]
    worst = 0.0
    for b in range(B):
        for h in range(H):
            ref = oracle.bob_head(*oracle_inputs(ins, b, h), scale, causal=True)
            for k in range(4):
                e = rel_fro(to_f64(outs[k][b, h]), ref[k])
                worst = max(worst, e)
                assert e <= tol, f"{label} b={b} h={h} output {k}: rel {e:.3e} > {tol}"
    return worst


@pytest.mark.parametrize("widx", [0, 1])
def test_causal_workload_full_oracle(widx):
    w = WORKLOADS[widx]
    say(f"[causal] workload {w.name} full oracle")
    ins = workload_inputs(w)
    outs = gpu_bob(ins, causal=True)
    worst = check_heads(ins, outs, w.scale, TOL[w.dtype], w.name)
    say(f"[causal] {w.name}: worst rel {worst:.3e}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [2, 33, 129, 200, 383, 520])
def test_causal_ragged_lengths(N, d, dtype):
    say(f"[causal] ragged N={N} d={d} {dtype}")
    ins = make_inputs(1, 2, N, d, dtype, seed=2000 + N + d)
    s = 1.0 / math.sqrt(d)
    outs = gpu_bob(ins, scale=s, causal=True)
    check_heads(ins, outs, s, TOL[dtype], f"causal N={N} d={d}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_causal_single_key(dtype):
    """N = 1 (masked or not, one key): gradQ, gradK, gradV are exactly zero and
    graddO = gV, reached up to float32 rounding (single_key_bounds derives the
    absolute bounds; a relative error against zero means nothing)."""
    ins = make_inputs(2, 1, 1, 64, dtype, seed=31)
    gq, gk, gv, gdo = gpu_bob(ins, causal=True)
    zero, gdo_err = single_key_bounds(ins, 1.0 / 8.0)
    assert float(gq.abs().max()) <= zero and float(gk.abs().max()) <= zero and float(gv.abs().max()) <= zero
    assert float((gdo - ins["gV"].float()).abs().max()) <= gdo_err


@pytest.mark.parametrize("scale", [-0.3, 0.0])
def test_causal_other_scales(scale):
    ins = make_inputs(1, 1, 300, 64, torch.float32, seed=91)
    outs = gpu_bob(ins, scale=scale, causal=True)
    check_heads(ins, outs, scale, 1e-4, f"causal scale={scale}")


def test_causal_first_row_closed_form():
    ins = make_inputs(1, 2, 1000, 64, torch.float32, seed=5)
    outs = gpu_bob(ins, causal=True)
    gq, gdo = to_f64(outs[0]), to_f64(outs[3])
    gv = to_f64(ins["gV"])
    assert np.abs(gq[:, :, 0]).max() <= 1e-6 * np.abs(gq).max()
    assert np.abs(gdo[:, :, 0] - gv[:, :, 0]).max() <= 1e-5 * np.abs(gv[:, :, 0]).max()


@pytest.fixture(scope="module")
def big_causal():
    w = WORKLOADS[3]
    say(f"[causal] workload {w.name} device runs (bf16 and fp32 paths)")
    ins = workload_inputs(w)
    out_bf = gpu_bob(ins, causal=True)
    out_f32 = gpu_bob(ins, dtype=torch.float32, causal=True)
    return w, ins, out_bf, out_f32


def test_causal_big_rows_vs_oracle(big_causal):
    w, ins, out_bf, out_f32 = big_causal
    g = torch.Generator().manual_seed(7)
    for h in range(w.H):
        k = int(torch.randint(1, w.N // 256 - 1, (1,), generator=g))
        for rows in (np.arange(256), np.arange(256 * k, 256 * (k + 1)), np.arange(w.N - 256, w.N)):
            xs = oracle_inputs(ins, 0, h)
            gq, gdo = oracle.bob_rows_head(*xs, w.scale, rows, causal=True)
            for name, outs, tol in (("bf16", out_bf, TOL[torch.bfloat16]), ("f32", out_f32, TOL[torch.float32])):
                e_q = rel_fro(to_f64(outs[0][0, h][rows]), gq)
                e_o = rel_fro(to_f64(outs[3][0, h][rows]), gdo)
                say(f"[causal] {w.name} h={h} rows {rows[0]}..: {name} gradQ {e_q:.2e} graddO {e_o:.2e}")
                assert e_q <= tol and e_o <= tol


def test_causal_big_consistency_and_key_shift(big_causal):
    w, _, out_bf, out_f32 = big_causal
    for k in range(4):
        e = rel_fro(to_f64(out_bf[k]), to_f64(out_f32[k]))
        assert e <= TOL[torch.bfloat16], f"output {k}: bf16 vs fp32 {e:.3e}"
    for outs, tol in ((out_f32, 1e-4), (out_bf, 2e-2)):
        for k in (1, 2):
            x = to_f64(outs[k])
            cs = np.linalg.norm(x.sum(axis=2))
            assert cs <= tol * np.linalg.norm(x), f"output {k}: colsum {cs:.3e}"


@pytest.mark.parametrize("N", [1, 77, 300])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_causal_rowstats_vs_oracle(N, dtype):
    ins = make_inputs(1, 2, N, 64, dtype, seed=400 + N)
    dev = [ins[k].to("cuda") for k in NAMES]
    stats = fb.rowstats(*dev, causal=True)
    torch.cuda.synchronize()
    tol = 1e-4 if dtype == torch.float32 else 2e-2
    for h in range(2):
        ref = oracle.row_stats_head(*oracle_inputs(ins, 0, h), 1.0 / 8.0, causal=True)
        for k in range(4):
            got = to_f64(stats[k][0, h].cpu())
            e = np.abs(got - ref[k]).max() / max(1.0, np.abs(ref[k]).max())
            assert e <= tol, f"N={N} stat {k}: {e:.3e}"
