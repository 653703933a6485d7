"""Parity of the HIP BoB path (through the C ABI) with the fp64 oracle.

Tolerances (max relative Frobenius error over the four outputs): 1e-4 for
fp32 inputs, 2e-2 for bf16 inputs with fp32 accumulation.

  * the 128/4096/16384-length workloads: full oracle, every output element
    (the 16384 one per head, to bound host time);
  * the 65536/262144-length workloads, in the launch configuration the
    benchmark times: oracle rows for a sampled block of 256 queries per head
    (gradQ, graddO are row-local), fp32-vs-bf16 self-consistency of all four
    outputs on the device, key-shift invariance (column sums of gradK and
    gradV vanish) and Hessian symmetry over two cotangent sets;
  * ragged lengths spanning several tiles, both head dims and both dtypes;
  * degenerate cases: zero cotangents, zero dO, a single key, empty input.
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


def check_all_heads(w_ins, outs, scale, tol, label, block=None):
    B, H = w_ins["Q"].shape[:2]
    worst = 0.0
    for b in range(B):
        for h in range(H):
            xs = oracle_inputs(w_ins, b, h)
            if block is None:
                ref = oracle.bob_head(*xs, scale)
            else:
                ref = oracle.bob_blocked_head(*xs, scale, block=block)
            for k in range(4):
                e = rel_fro(to_f64(outs[k][b, h]), ref[k])
                worst = max(worst, e)
                assert e <= tol, f"{label} b={b} h={h} output {k}: rel {e:.3e} > {tol}"
    return worst


@pytest.mark.parametrize("widx", [0, 1])
def test_workload_full_oracle(widx):
    w = WORKLOADS[widx]
    say(f"[parity] workload {w.name} full oracle")
    ins = workload_inputs(w)
    outs = gpu_bob(ins)
    worst = check_all_heads(ins, outs, w.scale, TOL[w.dtype], w.name)
    say(f"[parity] {w.name}: worst rel {worst:.3e}")


@pytest.fixture(scope="module")
def w2_outputs():
    w = WORKLOADS[2]
    say(f"[parity] workload {w.name} device run")
    ins = workload_inputs(w)
    return w, ins, gpu_bob(ins)


@pytest.mark.parametrize("head", range(8))
def test_workload_16384_per_head(w2_outputs, head):
    w, ins, outs = w2_outputs
    xs = oracle_inputs(ins, 0, head)
    ref = oracle.bob_blocked_head(*xs, w.scale, block=2048)
    for k in range(4):
        e = rel_fro(to_f64(outs[k][0, head]), ref[k])
        assert e <= TOL[w.dtype], f"head {head} output {k}: rel {e:.3e}"


def sampled_block(N, seed):
    g = torch.Generator().manual_seed(seed + 1)
    k = int(torch.randint(0, N // 256, (1,), generator=g))
    return np.arange(256 * k, 256 * (k + 1))


@pytest.fixture(scope="module", params=[3, 4])
def big(request):
    widx = request.param
    w = WORKLOADS[widx]
    say(f"[parity] workload {w.name} device runs (bf16 and fp32 paths)")
    ins = workload_inputs(w)
    out_bf = gpu_bob(ins)
    out_f32 = gpu_bob(ins, dtype=torch.float32)  # same bf16-exact values, fp32 path
    return widx, w, ins, out_bf, out_f32


def test_big_sampled_rows_vs_oracle(big):
    widx, w, ins, out_bf, out_f32 = big
    for h in range(w.H):
        rows = sampled_block(w.N, widx + h)
        xs = oracle_inputs(ins, 0, h)
        gq, gdo = oracle.bob_rows_head(*xs, w.scale, rows)
        for name, outs, tol in (("bf16", out_bf, TOL[torch.bfloat16]), ("f32", out_f32, TOL[torch.float32])):
            e_q = rel_fro(to_f64(outs[0][0, h][rows]), gq)
            e_o = rel_fro(to_f64(outs[3][0, h][rows]), gdo)
            say(f"[parity] {w.name} h={h} rows {rows[0]}..: {name} gradQ {e_q:.2e} graddO {e_o:.2e}")
            assert e_q <= tol and e_o <= tol


def test_big_bf16_matches_fp32_path(big):
    _, w, _, out_bf, out_f32 = big
    for k in range(4):
        e = rel_fro(to_f64(out_bf[k]), to_f64(out_f32[k]))
        assert e <= TOL[torch.bfloat16], f"output {k}: {e:.3e}"


def test_big_key_shift_invariance(big):
    _, w, _, out_bf, out_f32 = big
    for outs, tol in ((out_f32, 1e-4), (out_bf, 2e-2)):
        for k in (1, 2):  # gradK, gradV: columns sum to zero per head
            x = to_f64(outs[k])
            cs = np.linalg.norm(x.sum(axis=2))
            assert cs <= tol * np.linalg.norm(x), f"output {k}: colsum {cs:.3e}"


def test_big_hessian_symmetry(big):
    widx, w, ins, _, out_f32 = big
    say(f"[parity] {w.name} Hessian symmetry (second cotangent set, fp32 path)")
    other = make_inputs(w.B, w.H, w.N, w.d, w.dtype, seed=widx + 100)
    ins2 = dict(ins)
    for k in ("gQ", "gK", "gV"):
        ins2[k] = other[k]
    out2 = gpu_bob(ins2, dtype=torch.float32)
    g = [to_f64(ins[k].float()) for k in ("gQ", "gK", "gV")]
    hv = [to_f64(ins2[k].float()) for k in ("gQ", "gK", "gV")]
    lhs = sum(float(np.sum(a * to_f64(b))) for a, b in zip(hv, out_f32[:3]))
    rhs = sum(float(np.sum(a * to_f64(b))) for a, b in zip(g, out2[:3]))
    norm = math.sqrt(sum(float(np.sum(a * a)) for a in hv)) * math.sqrt(
        sum(float(np.sum(to_f64(b) ** 2)) for b in out_f32[:3]))
    say(f"[parity] symmetry lhs {lhs:.6e} rhs {rhs:.6e} scale {norm:.3e}")
    assert abs(lhs - rhs) <= 1e-4 * norm


RAGGED = [2, 31, 33, 100, 129, 200, 383]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", RAGGED)
def test_ragged_lengths(N, d, dtype):
    say(f"[parity] ragged N={N} d={d} {dtype}")
    ins = make_inputs(1, 2, N, d, dtype, seed=1000 + N + d)
    s = 1.0 / math.sqrt(d)
    outs = gpu_bob(ins, scale=s)
    check_all_heads(ins, outs, s, TOL[dtype], f"N={N} d={d}")


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.9])
def test_other_scales(scale):
    say(f"[parity] scale={scale}")
    ins = make_inputs(1, 1, 257, 64, torch.float32, seed=77)
    outs = gpu_bob(ins, scale=scale)
    check_all_heads(ins, outs, scale, 1e-4, f"scale={scale}")


def test_zero_cotangents_give_exact_zeros():
    ins = make_inputs(1, 2, 300, 64, torch.bfloat16, seed=5)
    for k in ("gQ", "gK", "gV"):
        ins[k] = torch.zeros_like(ins[k])
    say("[parity] zero cotangents")
    outs = gpu_bob(ins)
    for o in outs:
        assert torch.count_nonzero(o) == 0


def test_zero_dO_zeroes_first_three_outputs():
    ins = make_inputs(1, 1, 256, 64, torch.bfloat16, seed=6)
    ins["dO"] = torch.zeros_like(ins["dO"])
    say("[parity] zero dO")
    gq, gk, gv, gdo = gpu_bob(ins)
    assert torch.count_nonzero(gq) == 0 and torch.count_nonzero(gk) == 0 and torch.count_nonzero(gv) == 0
    assert torch.count_nonzero(gdo) > 0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_single_key(d, dtype):
    """N = 1: P = 1, so gradQ, gradK, gradV are exactly zero and graddO = gV;
    the kernels reach them up to float32 rounding (single_key_bounds derives
    the absolute bounds; a relative error against zero means nothing)."""
    ins = make_inputs(2, 1, 1, d, dtype, seed=8 + d)
    say(f"[parity] N=1 d={d} {dtype}")
    gq, gk, gv, gdo = gpu_bob(ins)
    zero, gdo_err = single_key_bounds(ins, 1.0 / math.sqrt(d))
    assert float(gq.abs().max()) <= zero and float(gk.abs().max()) <= zero and float(gv.abs().max()) <= zero
    assert float((gdo - ins["gV"].float()).abs().max()) <= gdo_err


def test_empty_sequence_is_noop():
    ins = make_inputs(1, 2, 0, 64, torch.bfloat16, seed=9)
    say("[parity] N=0")
    outs = gpu_bob(ins)
    assert all(o.numel() == 0 for o in outs)


def test_bitwise_repeatable():
    """Every output element is accumulated in registers in a fixed order (no
    atomics), so two calls give identical bits."""
    ins = make_inputs(1, 2, 1024, 64, torch.bfloat16, seed=10)
    say("[parity] repeatability")
    a = gpu_bob(ins)
    b = gpu_bob(ins)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_nondefault_stream():
    ins = make_inputs(1, 1, 512, 64, torch.bfloat16, seed=11)
    ref = gpu_bob(ins)
    dev = [ins[k].cuda() for k in NAMES]
    s = torch.cuda.Stream()
    say("[parity] side stream")
    with torch.cuda.stream(s):
        out = fb.bob(*dev)
    s.synchronize()
    for x, y in zip(out, ref):
        assert rel_fro(to_f64(x), to_f64(y)) <= 1e-6


@pytest.mark.parametrize("widx", [0, 1])
def test_rowstats_vs_oracle(widx):
    w = WORKLOADS[widx]
    ins = workload_inputs(w)
    dev = [ins[k].cuda() for k in NAMES]
    say(f"[parity] rowstats {w.name}")
    lse, D, c, r = [to_f64(t) for t in fb.rowstats(*dev)]
    torch.cuda.synchronize()
    for b in range(w.B):
        for h in range(w.H):
            ref = oracle.row_stats_head(*oracle_inputs(ins, b, h), w.scale)
            for name, got, want in zip(("lse", "D", "c", "r"), (lse, D, c, r), ref):
                e = rel_fro(got[b, h], want)
                assert e <= 1e-4, f"{name} b={b} h={h}: {e:.3e}"


@pytest.mark.parametrize("N", [1, 70, 300])
def test_rowstats_ragged(N):
    ins = make_inputs(1, 1, N, 128, torch.float32, seed=20 + N)
    dev = [ins[k].cuda() for k in NAMES]
    s = 1.0 / math.sqrt(128)
    say(f"[parity] rowstats ragged N={N}")
    got = [to_f64(t)[0, 0] for t in fb.rowstats(*dev, scale=s)]
    ref = oracle.row_stats_head(*oracle_inputs(ins, 0, 0), s)
    for g, want in zip(got, ref):
        assert rel_fro(g, want) <= 1e-5


def test_no_n_by_n_memory():
    """The call allocates nothing: device free memory is unchanged around it."""
    w = WORKLOADS[4]
    ins = workload_inputs(w)
    dev = [ins[k].cuda() for k in NAMES]
    out = tuple(torch.empty(dev[0].shape, dtype=torch.float32, device="cuda") for _ in range(4))
    ws = torch.empty(fb.workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    say("[parity] memory bound at N=262144")
    fb.bob(*dev, out=out, workspace=ws)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free0 - free1 <= 64 << 20
    assert torch.isfinite(out[0]).all()
