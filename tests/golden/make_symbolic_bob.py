"""Writes symbolic_bob.json: exact BoB values for tiny inputs, by symbolic
differentiation (sympy) of the objective's own definition.

Source: "FlashBoB: I/O-Efficient Exact Backward-over-Backward for Softmax
Attention" (arXiv 2609.24089), Abstract: BoB is the exact gradient of a
scalar built from the first backward pass of softmax attention. Here that
scalar is written out from its definition with exact rational inputs:
  S = s Q K^T (causal: -inf above the diagonal), P = softmax_rows(S),
  O = P V, dP = dO V^T, D = rowsum(dO o O), dS = P o (dP - D),
  dQ = s dS K, dK = s dS^T Q, dV = P^T dO,
  L = <gQ, dQ> + <gK, dK> + <gV, dV>,
and sympy differentiates L with respect to every entry of Q, K, V and dO.
Each case also records the first backward itself, obtained independently
by differentiating the forward <dO, O> with respect to Q, K and V. A
grouped case has two query heads share one key/value head: the objective is
the sum over the heads, so the shared heads' gradients sum over the group
by construction. Values are evaluated to 30 significant digits. The script uses neither the
oracle nor the HIP path; it is the independent reference the oracle is
checked against (tests/test_oracle.py).

usage: python tests/golden/make_symbolic_bob.py   (rewrites symbolic_bob.json)
"""

import json
import os
import random

import sympy as sp

HERE = os.path.dirname(os.path.abspath(__file__))
CASES = [  # (name, N, d, scale, causal, seed, query heads per key/value head)
    ("n2d2_plain", 2, 2, sp.Rational(1, 2), False, 1, 1),
    ("n3d2_causal", 3, 2, sp.Rational(3, 5), True, 2, 1),
    ("n3d1_plain_negscale", 3, 1, sp.Rational(-7, 10), False, 3, 1),
    ("n2d2_grouped2_causal", 2, 2, sp.Rational(2, 3), True, 4, 2),
]


def rational_matrix(rng, n, d):
    return sp.Matrix(n, d, lambda i, j: sp.Rational(rng.randint(-12, 12), 8))


def head_terms(Q, K, V, dO, gQ, gK, gV, N, d, s, causal):
    """(L, <dO, O>) of one query head, written from the definitions."""
    S = s * Q * K.T
    P = sp.zeros(N, N)
    for i in range(N):
        visible = [j for j in range(N) if not (causal and j > i)]
        den = sum(sp.exp(S[i, j]) for j in visible)
        for j in visible:
            P[i, j] = sp.exp(S[i, j]) / den
    O = P * V
    dP = dO * V.T
    D = [sum(dO[i, c] * O[i, c] for c in range(d)) for i in range(N)]
    dS = sp.Matrix(N, N, lambda i, j: P[i, j] * (dP[i, j] - D[i]))
    dQ = s * dS * K
    dK = s * dS.T * Q
    dV = P.T * dO
    L = sum(gQ[i, c] * dQ[i, c] + gK[i, c] * dK[i, c] + gV[i, c] * dV[i, c] for i in range(N) for c in range(d))
    fwd = sum(dO[i, c] * O[i, c] for i in range(N) for c in range(d))
    return L, fwd


def bob_values(N, d, s, causal, rng, G):
    """Inputs, outputs and objective of G query heads sharing one key/value
    head (G = 1: plain multi-head); query-side tensors are [G][N][d]."""
    qside, kside = ("Q", "dO", "gQ"), ("K", "V", "gK", "gV")
    vals = {k: [rational_matrix(rng, N, d) for _ in range(G)] for k in qside}
    vals.update({k: [rational_matrix(rng, N, d)] for k in kside})
    sym = {k: [sp.Matrix(N, d, lambda i, j, k=k, h=h: sp.Symbol(f"{k}{h}_{i}_{j}")) for h in range(len(vals[k]))]
           for k in ("Q", "K", "V", "dO")}
    L, fwd = 0, 0
    for h in range(G):
        Lh, fh = head_terms(sym["Q"][h], sym["K"][0], sym["V"][0], sym["dO"][h], vals["gQ"][h], vals["gK"][0],
                            vals["gV"][0], N, d, s, causal)
        L, fwd = L + Lh, fwd + fh
    subs = {sym[k][h][i, j]: vals[k][h][i, j] for k in sym for h in range(len(sym[k]))
            for i in range(N) for j in range(d)}

    def grad(expr, k):
        return [[[sp.N(sp.diff(expr, M[i, j]).subs(subs), 30) for j in range(d)] for i in range(N)] for M in sym[k]]

    out = {"gradQ": grad(L, "Q"), "gradK": grad(L, "K"), "gradV": grad(L, "V"), "graddO": grad(L, "dO"),
           "dQ": grad(fwd, "Q"), "dK": grad(fwd, "K"), "dV": grad(fwd, "V")}
    return vals, out, sp.N(L.subs(subs), 30)


def main():
    cases = []
    for name, N, d, s, causal, seed, G in CASES:
        vals, out, L = bob_values(N, d, s, causal, random.Random(seed), G)
        cases.append({
            "name": name, "N": N, "d": d, "scale": str(s), "causal": causal, "group": G,
            # [heads][N][d]: query-side tensors have G heads, key/value-side one
            "inputs": {k: [[[str(x) for x in row] for row in m.tolist()] for m in ms] for k, ms in vals.items()},
            "objective": str(L),
            "outputs": {k: [[[str(x) for x in row] for row in m] for m in v] for k, v in out.items()},
        })
        print(f"{name}: L = {L}")
    doc = {"source": "FlashBoB: I/O-Efficient Exact Backward-over-Backward for Softmax Attention "
                     "(arXiv 2609.24089), Abstract; values by sympy differentiation of the objective's definition "
                     "(tests/golden/make_symbolic_bob.py)",
           "cases": cases}
    with open(os.path.join(HERE, "symbolic_bob.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
