"""Pins of the fp64 oracle against routes that do not share its arithmetic.

Each pin would fail on a plausible mistake in the oracle (a dropped term, a
wrong sign or index, a transposed operand); test_pins_catch_planted_mistakes
plants such mistakes in the oracle, on the CPU, and checks that they are caught.

Independent routes used:
  * torch.autograd on an attention forward written with torch ops (first
    derivatives for the finite-difference objective; second derivatives with
    create_graph for the whole BoB);
  * central finite differences of the scalar objective;
  * forward-mode JVP of attention (graddO is the JVP along the cotangents);
  * second derivatives of the forward along a line (quadratic form);
  * torch's scaled_dot_product_attention backward (special case gQ = gK = 0)
    and forward (the attention the oracle differentiates, plain and causal);
  * identities the mathematics fixes: Hessian symmetry, Euler identity,
    bilinearity, zero cotangents, N = 1, key-shift invariance.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import bob_oracle



@pytest.fixture(autouse=True)
def _float64_default():
    # the torch references here are built in float64; the default is set per
    # test and restored, so it does not leak into other test modules
    prev = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(prev)

SHAPES = [(1, 3), (5, 4), (33, 8), (64, 16)]


def rand_inputs(N, d, seed, qk=1.0):
    rng = np.random.default_rng(seed)
    xs = [rng.standard_normal((N, d)) for _ in range(7)]
    xs[0] *= qk
    xs[1] *= qk
    return xs


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


# ----------------------------------------------------------------------------
# independent torch routes (no oracle code)


def torch_attn(Q, K, V, scale):
    return torch.softmax(scale * Q @ K.T, dim=-1) @ V


def torch_first_backward(Q, K, V, dO, scale, create_graph):
    """(dQ, dK, dV) = gradient of <dO, attention(Q, K, V)> by torch.autograd."""
    f = torch.sum(dO * torch_attn(Q, K, V, scale))
    return torch.autograd.grad(f, (Q, K, V), create_graph=create_graph)


def torch_L(xs, scale):
    Q, K, V, dO, gQ, gK, gV = [torch.tensor(x, requires_grad=True) for x in xs]
    dQ, dK, dV = torch_first_backward(Q, K, V, dO, scale, create_graph=True)
    L = torch.sum(gQ * dQ) + torch.sum(gK * dK) + torch.sum(gV * dV)
    return L, (Q, K, V, dO)


def torch_bob(xs, scale):
    L, prim = torch_L(xs, scale)
    grads = torch.autograd.grad(L, prim, allow_unused=True)
    return [np.zeros(x.shape) if g is None else g.detach().numpy() for g, x in zip(grads, xs[:4])]


def L_value(xs, scale):
    """Objective through torch first derivatives only (no second order)."""
    Q, K, V, dO = [torch.tensor(x, requires_grad=True) for x in xs[:4]]
    dQ, dK, dV = torch_first_backward(Q, K, V, dO, scale, create_graph=False)
    gQ, gK, gV = [torch.tensor(x) for x in xs[4:]]
    return float(torch.sum(gQ * dQ) + torch.sum(gK * dK) + torch.sum(gV * dV))


# ----------------------------------------------------------------------------
# pins


@pytest.mark.parametrize("N,d", SHAPES)
def test_matches_autograd_double_backward(N, d):
    xs = rand_inputs(N, d, seed=10 * N + d)
    s = 1.0 / math.sqrt(d)
    got = oracle.bob_head(*xs, s)
    ref = torch_bob(xs, s)
    for g, r in zip(got, ref):
        if np.linalg.norm(r) == 0:
            assert np.abs(g).max() < 1e-12
        else:
            assert rel(g, r) < 1e-12


@pytest.mark.parametrize("N,d", [(5, 4), (33, 8)])
def test_central_finite_differences(N, d):
    xs = rand_inputs(N, d, seed=7 + N)
    s = 1.0 / math.sqrt(d)
    got = oracle.bob_head(*xs, s)
    rng = np.random.default_rng(99)
    h = 1e-5
    for k in range(4):  # Q, K, V, dO
        u = rng.standard_normal(xs[k].shape)
        xp = list(xs)
        xm = list(xs)
        xp[k] = xs[k] + h * u
        xm[k] = xs[k] - h * u
        fd = (L_value(xp, s) - L_value(xm, s)) / (2 * h)
        an = float(np.sum(got[k] * u))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (k, fd, an)


@pytest.mark.parametrize("N,d", SHAPES)
def test_graddO_is_forward_jvp(N, d):
    xs = rand_inputs(N, d, seed=3 * N + d)
    s = 1.0 / math.sqrt(d)
    _, _, _, graddO = oracle.bob_head(*xs, s)
    prim = tuple(torch.tensor(x) for x in xs[:3])
    tang = tuple(torch.tensor(x) for x in xs[4:])
    _, jvp = torch.func.jvp(lambda q, k, v: torch_attn(q, k, v, s), prim, tang)
    assert rel(graddO, jvp.numpy()) < 1e-12


@pytest.mark.parametrize("N,d", [(5, 4), (33, 8), (64, 16)])
def test_hessian_symmetry(N, d):
    xs = rand_inputs(N, d, seed=N + 5 * d)
    hs = rand_inputs(N, d, seed=N + 5 * d + 1)[4:]
    s = 1.0 / math.sqrt(d)
    bg = oracle.bob_head(*xs, s)
    bh = oracle.bob_head(*xs[:4], *hs, s)
    lhs = sum(np.sum(h * b) for h, b in zip(hs, bg[:3]))
    rhs = sum(np.sum(g * b) for g, b in zip(xs[4:], bh[:3]))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


@pytest.mark.parametrize("N,d", [(5, 4), (33, 8)])
def test_quadratic_form_is_second_derivative_of_forward(N, d):
    xs = rand_inputs(N, d, seed=11 * N + d)
    s = 1.0 / math.sqrt(d)
    Q, K, V, dO, gQ, gK, gV = [torch.tensor(x) for x in xs]
    gradQ, gradK, gradV, _ = oracle.bob_head(*xs, s)
    quad = np.sum(xs[4] * gradQ) + np.sum(xs[5] * gradK) + np.sum(xs[6] * gradV)
    t = torch.zeros((), requires_grad=True)
    f = torch.sum(dO * torch_attn(Q + t * gQ, K + t * gK, V + t * gV, s))
    (df,) = torch.autograd.grad(f, t, create_graph=True)
    (d2f,) = torch.autograd.grad(df, t)
    assert abs(float(d2f) - quad) <= 1e-10 * max(1.0, abs(quad))


@pytest.mark.parametrize("N,d", SHAPES)
def test_euler_identity(N, d):
    xs = rand_inputs(N, d, seed=2 * N + d)
    s = 1.0 / math.sqrt(d)
    _, _, _, graddO = oracle.bob_head(*xs, s)
    L = L_value(xs, s)
    assert abs(np.sum(xs[3] * graddO) - L) <= 1e-12 * max(1.0, abs(L))


def test_bilinearity():
    xs = rand_inputs(33, 8, seed=1)
    s = 1.0 / math.sqrt(8)
    base = oracle.bob_head(*xs, s)
    x2 = list(xs)
    x2[3] = 2.0 * xs[3]
    two = oracle.bob_head(*x2, s)
    for k in range(3):
        assert rel(two[k], 2.0 * base[k]) < 1e-13
    assert rel(two[3], base[3]) < 1e-13
    x3 = list(xs)
    for k in range(4, 7):
        x3[k] = 3.0 * xs[k]
    three = oracle.bob_head(*x3, s)
    for k in range(4):
        assert rel(three[k], 3.0 * base[k]) < 1e-13


def test_zero_cotangents_and_zero_dO():
    xs = rand_inputs(33, 8, seed=2)
    s = 1.0 / math.sqrt(8)
    z = list(xs)
    for k in range(4, 7):
        z[k] = np.zeros_like(xs[k])
    for out in oracle.bob_head(*z, s):
        assert np.all(out == 0.0)
    z = list(xs)
    z[3] = np.zeros_like(xs[3])
    gq, gk, gv, gdo = oracle.bob_head(*z, s)
    assert np.all(gq == 0) and np.all(gk == 0) and np.all(gv == 0)
    assert np.linalg.norm(gdo) > 0


@pytest.mark.parametrize("N,d", [(5, 4), (64, 16)])
def test_gQ_gK_zero_reduces_to_textbook_attention_backward(N, d):
    xs = rand_inputs(N, d, seed=17 + N)
    xs[4] = np.zeros_like(xs[4])
    xs[5] = np.zeros_like(xs[5])
    s = 1.0 / math.sqrt(d)
    gq, gk, gv, gdo = oracle.bob_head(*xs, s)
    Q, K, gV, dO = [torch.tensor(x, requires_grad=True) for x in (xs[0], xs[1], xs[6], xs[3])]
    O = torch.nn.functional.scaled_dot_product_attention(
        Q[None, None], K[None, None], gV[None, None], scale=s)[0, 0]
    dq, dk = torch.autograd.grad(torch.sum(dO * O), (Q, K))
    assert rel(gq, dq.numpy()) < 1e-12
    assert rel(gk, dk.numpy()) < 1e-12
    assert np.all(gv == 0.0)
    assert rel(gdo, O.detach().numpy()) < 1e-12


def test_single_key_gives_zero_gradients_and_gV():
    xs = rand_inputs(1, 8, seed=4)
    gq, gk, gv, gdo = oracle.bob_head(*xs, 0.35)
    # P = 1 exactly, so dS = dP - D and A = G - c vanish up to the rounding of
    # two fp64 dot products of the same vectors
    tol = 1e-14 * max(np.abs(x).max() for x in xs) ** 3
    assert np.abs(gq).max() < tol and np.abs(gk).max() < tol and np.abs(gv).max() < tol
    assert np.abs(gdo - xs[6]).max() < tol


@pytest.mark.parametrize("N,d", SHAPES)
def test_key_shift_invariance_column_sums(N, d):
    xs = rand_inputs(N, d, seed=5 * N + d)
    gq, gk, gv, _ = oracle.bob_head(*xs, 1.0 / math.sqrt(d))
    scale_k = max(1.0, np.abs(gk).max())
    scale_v = max(1.0, np.abs(gv).max())
    assert np.abs(gk.sum(axis=0)).max() < 1e-12 * N * scale_k
    assert np.abs(gv.sum(axis=0)).max() < 1e-12 * N * scale_v


@pytest.mark.parametrize("N,d,block", [(33, 8, 7), (64, 16, 16), (64, 16, 64)])
def test_row_stats_three_routes(N, d, block):
    xs = rand_inputs(N, d, seed=N * d)
    s = 1.0 / math.sqrt(d)
    lse, D, c, r = oracle.row_stats_head(*xs, s)
    D2, c2, r2 = oracle.row_stats_closed_forms_head(*xs, s)
    lse3, D3, c3, r3 = oracle.row_stats_online_head(*xs, s, block)
    S = s * xs[0] @ xs[1].T
    lse_lib = np.logaddexp.reduce(S, axis=1)
    for a, b in ((lse, lse_lib), (lse3, lse_lib), (D, D2), (D, D3), (c, c2), (c, c3), (r, r2), (r, r3)):
        assert np.abs(a - b).max() < 1e-12 * max(1.0, np.abs(b).max())


def test_blocked_and_row_forms_match_full():
    xs = rand_inputs(64, 8, seed=9)
    s = 1.0 / math.sqrt(8)
    full = oracle.bob_head(*xs, s)
    blk = oracle.bob_blocked_head(*xs, s, block=24)
    for a, b in zip(blk, full):
        assert rel(a, b) < 1e-13
    rows = np.arange(16, 40)
    gq, gdo = oracle.bob_rows_head(*xs, s, rows)
    assert rel(gq, full[0][rows]) < 1e-13
    assert rel(gdo, full[3][rows]) < 1e-13


def test_batched_wrappers_loop_heads():
    rng = np.random.default_rng(0)
    xs = [rng.standard_normal((2, 3, 17, 4)) for _ in range(7)]
    out = oracle.bob(*xs, 0.5)
    outb = oracle.bob_blocked(*xs, 0.5, block=5)
    for b in range(2):
        for h in range(3):
            ref = oracle.bob_head(*[x[b, h] for x in xs], 0.5)
            for k in range(4):
                assert rel(out[k][b, h], ref[k]) < 1e-14
                assert rel(outb[k][b, h], ref[k]) < 1e-13


# ----------------------------------------------------------------------------
# the pins above catch plausible mistakes (planted in the oracle, CPU only)

MUTATIONS = {
    "drop_P_H_term": lambda t: t.update(dS2=t["dS"] * (t["G"] - t["c"])),
    "no_centering_c": lambda t: t.update(A=t["P"] * t["G"]),
    "r_sign": lambda t: t.update(dS2=t["dS"] * (t["G"] - t["c"]) + t["P"] * (t["H"] + t["r"])),
    "D_as_constant": lambda t: t.update(A=t["P"] * t["G"],
                                        dS2=t["dS"] * t["G"] + t["P"] * (t["H"] - t["r"])),
    "LSE_as_constant": lambda t: t.update(dS2=t["dS"] * (t["G"] - t["c"]) + t["P"] * t["H"]),
    "transposed_G": lambda t: t.update(dS2=t["dS"] * (t["G"].T - t["c"]) + t["P"] * (t["H"] - t["r"])),
    "H_from_V": lambda t: t.update(H=t["dP"]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    N, d = 16, 4
    xs = rand_inputs(N, d, seed=123)
    s = 1.0 / math.sqrt(d)
    orig = bob_oracle._tiles

    def mutated(*a, **k):
        t = orig(*a, **k)
        if name == "H_from_V":
            MUTATIONS[name](t)
            t["dS2"] = t["dS"] * (t["G"] - t["c"]) + t["P"] * (t["H"] - t["r"])
        else:
            MUTATIONS[name](t)
        return t

    monkeypatch.setattr(bob_oracle, "_tiles", mutated)
    got = oracle.bob_head(*xs, s)
    ref = torch_bob(xs, s)
    worst = max(rel(g, r) for g, r in zip(got, ref))
    assert worst > 1e-3, f"mutation {name} not caught (worst rel {worst})"


# ----------------------------------------------------------------------------
# causal masking: query i attends to keys j <= i (a reading beyond the
# abstract). Independent routes: torch autograd through a masked torch
# attention, finite differences, and rows whose result is fixed in closed form.


def torch_attn_causal(Q, K, V, scale):
    N = Q.shape[0]
    mask = torch.ones(N, K.shape[0], dtype=torch.bool).triu(1)  # key j > query i
    S = (scale * Q @ K.T).masked_fill(mask, float("-inf"))
    return torch.softmax(S, dim=-1) @ V


def torch_bob_causal(xs, scale):
    Q, K, V, dO, gQ, gK, gV = [torch.tensor(x, requires_grad=True) for x in xs]
    f = torch.sum(dO * torch_attn_causal(Q, K, V, scale))
    dQ, dK, dV = torch.autograd.grad(f, (Q, K, V), create_graph=True)
    L = torch.sum(gQ * dQ) + torch.sum(gK * dK) + torch.sum(gV * dV)
    grads = torch.autograd.grad(L, (Q, K, V, dO), allow_unused=True)
    return [np.zeros(x.shape) if g is None else g.detach().numpy() for g, x in zip(grads, xs[:4])]


def L_value_causal(xs, scale):
    Q, K, V, dO = [torch.tensor(x, requires_grad=True) for x in xs[:4]]
    f = torch.sum(dO * torch_attn_causal(Q, K, V, scale))
    dQ, dK, dV = torch.autograd.grad(f, (Q, K, V))
    gQ, gK, gV = [torch.tensor(x) for x in xs[4:]]
    return float(torch.sum(gQ * dQ) + torch.sum(gK * dK) + torch.sum(gV * dV))


@pytest.mark.parametrize("N,d", [(1, 3), (5, 4), (33, 8), (64, 16)])
def test_causal_matches_autograd_double_backward(N, d):
    xs = rand_inputs(N, d, seed=17 * N + d)
    s = 1.0 / math.sqrt(d)
    got = oracle.bob_head(*xs, s, causal=True)
    ref = torch_bob_causal(xs, s)
    for g, r in zip(got, ref):
        if np.linalg.norm(r) == 0:
            assert np.abs(g).max() < 1e-12
        else:
            assert rel(g, r) < 1e-12


def test_causal_central_finite_differences():
    N, d = 17, 6
    xs = rand_inputs(N, d, seed=71)
    s = 0.4
    got = oracle.bob_head(*xs, s, causal=True)
    rng = np.random.default_rng(5)
    h = 1e-5
    for k in range(4):
        u = rng.standard_normal(xs[k].shape)
        xp, xm = list(xs), list(xs)
        xp[k] = xs[k] + h * u
        xm[k] = xs[k] - h * u
        fd = (L_value_causal(xp, s) - L_value_causal(xm, s)) / (2 * h)
        an = float(np.sum(got[k] * u))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (k, fd, an)


def test_causal_first_and_last_rows():
    # row 0 sees key 0 alone: P = 1, so dS = A = dS2 = 0 on that row and
    # gradQ_0 = 0, graddO_0 = gV_0 exactly; the last row sees every key, so
    # its gradQ and graddO equal the unmasked ones
    N, d = 29, 8
    xs = rand_inputs(N, d, seed=8)
    s = 0.3
    gq, gk, gv, gdo = oracle.bob_head(*xs, s, causal=True)
    assert np.abs(gq[0]).max() < 1e-14
    assert np.abs(gdo[0] - xs[6][0]).max() < 1e-14
    fq, fk, fv, fdo = oracle.bob_head(*xs, s)
    assert rel(gq[N - 1], fq[N - 1]) < 1e-13
    assert rel(gdo[N - 1], fdo[N - 1]) < 1e-13
    # the last key is seen by the last query only, so its gradK / gradV rows
    # come from that single (P = softmax weight) entry and differ from the
    # unmasked ones
    assert rel(gk[N - 1], fk[N - 1]) > 1e-3


def test_causal_hessian_symmetry_and_forms():
    N, d = 33, 8
    xs = rand_inputs(N, d, seed=41)
    hs = rand_inputs(N, d, seed=42)[4:]
    s = 1.0 / math.sqrt(d)
    bg = oracle.bob_head(*xs, s, causal=True)
    bh = oracle.bob_head(*xs[:4], *hs, s, causal=True)
    lhs = sum(np.sum(h * b) for h, b in zip(hs, bg[:3]))
    rhs = sum(np.sum(g * b) for g, b in zip(xs[4:], bh[:3]))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    # row-blocked, row-sampled and online forms are exact restrictions
    bb = oracle.bob_blocked_head(*xs, s, block=10, causal=True)
    assert max(rel(a, b) for a, b in zip(bb, bg)) < 1e-13
    rows = np.array([0, 7, 32])
    rq, rdo = oracle.bob_rows_head(*xs, s, rows, causal=True)
    assert rel(rq, bg[0][rows]) < 1e-13 and rel(rdo, bg[3][rows]) < 1e-13
    direct = oracle.row_stats_head(*xs, s, causal=True)
    online = oracle.row_stats_online_head(*xs, s, block=8, causal=True)
    closed = oracle.row_stats_closed_forms_head(*xs, s, causal=True)
    for a, b in zip(direct, online):
        assert rel(a, b) < 1e-12
    for a, b in zip(direct[1:], closed):
        assert rel(a, b) < 1e-12


@pytest.mark.parametrize("variant", ["diagonal_masked", "transposed_mask"])
def test_causal_pins_catch_planted_mask_mistakes(variant, monkeypatch):
    N, d = 16, 4
    xs = rand_inputs(N, d, seed=321)
    s = 0.5

    def mask(S, qidx, causal):
        if not causal:
            return S
        q = np.asarray(qidx).reshape(-1, 1)
        k = np.arange(S.shape[1]).reshape(1, -1)
        bad = (k >= q) if variant == "diagonal_masked" else (k < q)
        # keep at least one key per row so the softmax stays finite
        bad[:, 0] = bad[:, 0] & (q[:, 0] > 0) if variant == "diagonal_masked" else bad[:, 0]
        if variant == "diagonal_masked":
            bad[0, 0] = False
        return np.where(bad, -np.inf, S)

    monkeypatch.setattr(bob_oracle, "_mask_scores", mask)
    got = oracle.bob_head(*xs, s, causal=True)
    ref = torch_bob_causal(xs, s)
    worst = max(rel(g, r) for g, r in zip(got, ref))
    assert worst > 1e-3, f"planted {variant} not caught (worst rel {worst})"


# ----------------------------------------------------------------------------
# grouped key/value heads (GQA / MQA): query head h uses key/value head
# h // (H / Hkv). Independent route: torch autograd through a torch attention
# whose K, V are expanded with repeat_interleave (gradients flow back to the
# shared heads).


def torch_bob_gqa(xs, scale, causal):
    Q, K, V, dO, gQ, gK, gV = [torch.tensor(x, requires_grad=True) for x in xs]
    G = Q.shape[1] // K.shape[1]
    Ke, Ve = K.repeat_interleave(G, dim=1), V.repeat_interleave(G, dim=1)
    S = scale * Q @ Ke.transpose(-1, -2)
    if causal:
        N = Q.shape[2]
        S = S.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    f = torch.sum(dO * (torch.softmax(S, dim=-1) @ Ve))
    dQ, dK, dV = torch.autograd.grad(f, (Q, K, V), create_graph=True)
    L = torch.sum(gQ * dQ) + torch.sum(gK * dK) + torch.sum(gV * dV)
    grads = torch.autograd.grad(L, (Q, K, V, dO))
    return [g.detach().numpy() for g in grads]


@pytest.mark.parametrize("H,Hkv", [(4, 2), (3, 1), (2, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_matches_autograd(H, Hkv, causal):
    rng = np.random.default_rng(H * 10 + Hkv + causal)
    B, N, d = 2, 9, 4
    q_shape, kv_shape = (B, H, N, d), (B, Hkv, N, d)
    xs = [rng.standard_normal(s) for s in (q_shape, kv_shape, kv_shape, q_shape, q_shape, kv_shape, kv_shape)]
    got = oracle.bob_gqa(*xs, 0.45, causal=causal)
    ref = torch_bob_gqa(xs, 0.45, causal)
    for g, r in zip(got, ref):
        assert rel(g, r) < 1e-12
    blocked = oracle.bob_gqa(*xs, 0.45, causal=causal, block=4)
    for g, r in zip(blocked, got):
        assert rel(g, r) < 1e-13


def test_gqa_planted_mistake_is_caught(monkeypatch):
    # taking only the group's first query head for gradK, gradV (instead of
    # the sum over the group) must fail the autograd pin
    rng = np.random.default_rng(3)
    B, H, Hkv, N, d = 1, 4, 2, 7, 4
    q_shape, kv_shape = (B, H, N, d), (B, Hkv, N, d)
    xs = [rng.standard_normal(s) for s in (q_shape, kv_shape, kv_shape, q_shape, q_shape, kv_shape, kv_shape)]
    ref = torch_bob_gqa(xs, 0.5, False)
    orig = bob_oracle.bob_head
    calls = {"n": 0}

    def first_only(*a, **k):
        out = orig(*a, **k)
        calls["n"] += 1
        if calls["n"] % 2 == 0:  # the group's second head contributes nothing to gradK, gradV
            return out[0], np.zeros_like(out[1]), np.zeros_like(out[2]), out[3]
        return out

    monkeypatch.setattr(bob_oracle, "bob_head", first_only)
    got = oracle.bob_gqa(*xs, 0.5)
    assert max(rel(g, r) for g, r in zip(got, ref)) > 1e-3


# ----------------------------------------------------------------------------
# the first backward itself (returned by the library on request): pinned
# against torch autograd of <dO, attention(Q, K, V)>, with and without the
# causal mask


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("N,d", [(1, 3), (6, 4), (33, 8)])
def test_first_backward_matches_autograd(N, d, causal):
    xs = rand_inputs(N, d, seed=400 + N + d + causal)
    s = 0.35
    got = oracle.attention_backward(*xs[:4], s, causal=causal)
    Q, K, V = [torch.tensor(x, requires_grad=True) for x in xs[:3]]
    dO = torch.tensor(xs[3])
    attn = torch_attn_causal(Q, K, V, s) if causal else torch_attn(Q, K, V, s)
    ref = torch.autograd.grad(torch.sum(dO * attn), (Q, K, V))
    for g, r in zip(got, ref):
        r = r.numpy()
        if np.linalg.norm(r) == 0:
            assert np.abs(g).max() < 1e-13
        else:
            assert rel(g, r) < 1e-12


def test_first_backward_batched_gqa_matches_autograd():
    rng = np.random.default_rng(77)
    B, H, Hkv, N, d = 2, 4, 2, 7, 4
    Q, dO = rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, d))
    K, V = rng.standard_normal((B, Hkv, N, d)), rng.standard_normal((B, Hkv, N, d))
    for causal in (False, True):
        got = oracle.attention_backward_batched(Q, K, V, dO, 0.4, causal=causal)
        tq, tk, tv = [torch.tensor(x, requires_grad=True) for x in (Q, K, V)]
        S = 0.4 * tq @ tk.repeat_interleave(2, dim=1).transpose(-1, -2)
        if causal:
            S = S.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        out = torch.softmax(S, dim=-1) @ tv.repeat_interleave(2, dim=1)
        ref = torch.autograd.grad(torch.sum(torch.tensor(dO) * out), (tq, tk, tv))
        for g, r in zip(got, ref):
            assert rel(g, r.numpy()) < 1e-12


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_first_backward_rows_match_autograd(causal):
    # the row form (for sampled rows of long sequences) against autograd,
    # on rows that include the first and last (the causal extremes)
    xs = rand_inputs(40, 6, seed=91 + causal)
    s = 0.3
    rows = np.array([0, 1, 17, 38, 39])
    got = oracle.attention_backward_rows_head(*xs[:4], s, rows, causal=causal)
    Q, K, V = [torch.tensor(x, requires_grad=True) for x in xs[:3]]
    attn = torch_attn_causal(Q, K, V, s) if causal else torch_attn(Q, K, V, s)
    ref = torch.autograd.grad(torch.sum(torch.tensor(xs[3]) * attn), Q)[0].numpy()[rows]
    assert rel(got, ref) < 1e-12
    if causal:
        assert np.abs(got[0]).max() < 1e-14  # one visible key: dS = 0


# ----------------------------------------------------------------------------
# exact values by symbolic differentiation of the objective's definition
# (tests/golden/symbolic_bob.json, written by tests/golden/make_symbolic_bob.py
# with sympy: no oracle code involved)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "symbolic_bob.json")


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_oracle_matches_symbolic_differentiation(case):
    # BoB outputs and objective (grouped case: through bob_gqa) and the first
    # backward (sympy differentiated the forward <dO, O>, not the backward
    # formulas) against the exact values
    from fractions import Fraction

    def arr(heads):  # [heads][N][d] strings -> [1, heads, N, d] float64
        return np.array([[[[float(Fraction(x)) for x in r] for r in m] for m in heads]])

    x = {k: arr(case["inputs"][k]) for k in ("Q", "K", "V", "dO", "gQ", "gK", "gV")}
    xs = [x[k] for k in ("Q", "K", "V", "dO", "gQ", "gK", "gV")]
    s = float(Fraction(case["scale"]))
    causal = case["causal"]
    got = list(oracle.bob_gqa(*xs, s, causal=causal))
    got += list(oracle.attention_backward_batched(*xs[:4], s, causal=causal))
    for k, name in enumerate(("gradQ", "gradK", "gradV", "graddO", "dQ", "dK", "dV")):
        want = arr(case["outputs"][name])
        assert got[k].shape == want.shape, name
        assert np.abs(got[k] - want).max() <= 1e-12 * max(1.0, np.abs(want).max()), name
    if case["group"] == 1:
        h = [x[k][0, 0] for k in ("Q", "K", "V", "dO", "gQ", "gK", "gV")]
        L = oracle.bob_objective(*h, s, causal=causal)
        assert abs(L - float(case["objective"])) <= 1e-12 * max(1.0, abs(float(case["objective"])))


# ----------------------------------------------------------------------------
# the attention forward itself (the function whose derivatives BoB takes)


@pytest.mark.parametrize("N,d", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_attention_forward_matches_sdpa(N, d, causal):
    """oracle.attention_forward against torch's scaled_dot_product_attention in
    float64 (a library routine for the same definition, softmax(s Q K^T) V)."""
    Q, K, V = rand_inputs(N, d, seed=31 + N + d)[:3]
    s = 0.7 / math.sqrt(d)
    t = [torch.tensor(x)[None, None] for x in (Q, K, V)]
    ref = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=causal, scale=s)[0, 0].numpy()
    assert rel(oracle.attention_forward(Q, K, V, s, causal=causal), ref) < 1e-13


def test_attention_forward_closed_forms():
    """Special cases with answers that need no library: one key returns V;
    Q = 0 makes every score equal, so each row averages the values it sees
    (all rows plainly, rows 0..i causally); a large scale turns the softmax
    into a selection of the best-matching key."""
    rng = np.random.default_rng(5)
    d = 6
    K1, V1 = rng.standard_normal((1, d)), rng.standard_normal((1, d))
    Q1 = rng.standard_normal((1, d))
    assert np.allclose(oracle.attention_forward(Q1, K1, V1, 0.3), V1, rtol=0, atol=1e-15)
    N = 7
    K, V = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    Z = np.zeros((N, d))
    assert np.allclose(oracle.attention_forward(Z, K, V, 0.5), np.tile(V.mean(axis=0), (N, 1)), atol=1e-14)
    running = np.cumsum(V, axis=0) / np.arange(1, N + 1)[:, None]
    assert np.allclose(oracle.attention_forward(Z, K, V, 0.5, causal=True), running, atol=1e-14)
    # orthogonal keys, each query a multiple of one key: the selection is exact
    # up to exp(-scale * gap) ~ 1e-43
    Kd = np.eye(N, d) * 3.0
    perm = np.array([3, 0, 5, 1, 4, 2, 0])
    Qs = Kd[perm] if d >= N else None
    if Qs is not None:
        got = oracle.attention_forward(Qs, Kd, V, 100.0)
        assert np.allclose(got, V[perm], atol=1e-12)


@pytest.mark.parametrize("variant", ["softmax_over_queries", "no_mask", "mask_off_by_one", "V_rows_permuted"])
def test_attention_forward_pins_catch_planted_mistakes(variant, monkeypatch):
    """Each planted mistake in the forward (written into the oracle, on the
    CPU) fails the pins above."""
    orig_mask = bob_oracle._mask_scores
    orig_softmax = bob_oracle.softmax_rows
    if variant == "softmax_over_queries":
        monkeypatch.setattr(bob_oracle, "softmax_rows", lambda S: orig_softmax(np.asarray(S).T).T)
    elif variant == "no_mask":
        monkeypatch.setattr(bob_oracle, "_mask_scores", lambda S, qidx, causal: S)
    elif variant == "mask_off_by_one":
        def shifted(S, qidx, causal):
            return orig_mask(S, np.asarray(qidx) + 1, causal) if causal else S
        monkeypatch.setattr(bob_oracle, "_mask_scores", shifted)
    Q, K, V = rand_inputs(9, 4, seed=77)[:3]
    if variant == "V_rows_permuted":
        # the mistake is an operand-order one: feed V with its rows reversed
        # through the real oracle and check the pin sees the difference
        V_used = V[::-1].copy()
    else:
        V_used = V
    s = 0.6
    t = [torch.tensor(x)[None, None] for x in (Q, K, V)]
    worst = 0.0
    for causal in (False, True):
        ref = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=causal, scale=s)[0, 0].numpy()
        worst = max(worst, rel(bob_oracle.attention_forward(Q, K, V_used, s, causal=causal), ref))
    assert not worst <= 1e-3, f"planted {variant} not caught (worst rel {worst})"
