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
The values are evaluated to 30 significant digits. The script uses neither the
oracle nor the HIP path; it is the independent reference the oracle is
checked against (tests/test_oracle.py).

usage: python tests/golden/make_symbolic_bob.py   (rewrites symbolic_bob.json)
"""

import json
import os
import random

import sympy as sp

HERE = os.path.dirname(os.path.abspath(__file__))
CASES = [  # (name, N, d, scale, causal, seed)
    ("n2d2_plain", 2, 2, sp.Rational(1, 2), False, 1),
    ("n3d2_causal", 3, 2, sp.Rational(3, 5), True, 2),
    ("n3d1_plain_negscale", 3, 1, sp.Rational(-7, 10), False, 3),
]


def rational_matrix(rng, n, d):
    return sp.Matrix(n, d, lambda i, j: sp.Rational(rng.randint(-12, 12), 8))


def bob_values(N, d, s, causal, rng):
    names = ("Q", "K", "V", "dO", "gQ", "gK", "gV")
    vals = {k: rational_matrix(rng, N, d) for k in names}
    sym = {k: sp.Matrix(N, d, lambda i, j, k=k: sp.Symbol(f"{k}_{i}_{j}")) for k in ("Q", "K", "V", "dO")}
    Q, K, V, dO = sym["Q"], sym["K"], sym["V"], sym["dO"]
    gQ, gK, gV = vals["gQ"], vals["gK"], vals["gV"]
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
    subs = {sym[k][i, j]: vals[k][i, j] for k in sym for i in range(N) for j in range(d)}
    out = {}
    for name, M in (("gradQ", Q), ("gradK", K), ("gradV", V), ("graddO", dO)):
        out[name] = [[sp.N(sp.diff(L, M[i, j]).subs(subs), 30) for j in range(d)] for i in range(N)]
    return vals, out, sp.N(L.subs(subs), 30)


def main():
    cases = []
    for name, N, d, s, causal, seed in CASES:
        vals, out, L = bob_values(N, d, s, causal, random.Random(seed))
        cases.append({
            "name": name, "N": N, "d": d, "scale": str(s), "causal": causal,
            "inputs": {k: [[str(x) for x in row] for row in m.tolist()] for k, m in vals.items()},
            "objective": str(L),
            "outputs": {k: [[str(x) for x in row] for row in v] for k, v in out.items()},
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
