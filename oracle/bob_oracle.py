"""Plain fp64 CPU oracle for the exact backward-over-backward (BoB) of softmax attention.

TEST INFRASTRUCTURE. This module is the checker, not the product: only the
tests, the smoke check and the benchmark's CPU-baseline leg may import it. It
shares no code with the HIP path and imports nothing from it.

Source: "FlashBoB: I/O-Efficient Exact Backward-over-Backward for Softmax
Attention" (arXiv 2609.24089), Abstract. The abstract states that:
  * BoB differentiates exactly through the first backward pass of attention,
    the pass FlashAttention already makes I/O-efficient;
  * the method is exact (no approximation), so its result is the plain
    mathematical second-order gradient, reached up to rounding order;
  * inside the softmax double backward two row-wise scalars fix every output
    through affine maps, which is what allows a two-pass tiled schedule.

The abstract names neither the scalar objective nor the two scalars. The
readings taken here (listed with the others in the design notes):
  * objective  L = <gQ, dQ> + <gK, dK> + <gV, dV>, where (dQ, dK, dV) is the
    textbook first backward of O = softmax(scale * Q K^T) V for upstream dO;
    outputs are dL/dQ, dL/dK, dL/dV, dL/ddO;
  * the two row scalars are  c = rowsum(P o G)  and
    r = rowsum(dS o G) + rowsum(P o H)  (G, H, dS defined below), next to the
    first-backward row scalar D = rowsum(dO o O);
  * LSE and D are functions of the inputs and carry gradient (they are not
    stop-gradient constants).

Every function works per head on 2-D arrays [N, d] in float64 and
materialises the N x N quantities; the batched wrappers loop over [B, H].

Causal masking (a reading beyond the abstract, which does not treat masks):
with causal=True query i attends to keys j <= i only. The masked scores are
-inf constants, so P, dS, A and dS2 vanish there and no gradient flows
through them; everything else is unchanged.
"""

import numpy as np

__all__ = [
    "softmax_rows",
    "attention_forward",
    "attention_backward",
    "bob_objective",
    "bob_head",
    "bob",
    "row_stats_head",
    "row_stats_closed_forms_head",
    "row_stats_online_head",
    "bob_rows_head",
    "bob_blocked_head",
    "bob_blocked",
    "bob_gqa",
    "attention_backward_batched",
    "attention_backward_rows_head",
]


def _f64(*xs):
    return [np.asarray(x, dtype=np.float64) for x in xs]


def _mask_scores(S, qidx, causal):
    """Scores with the causal mask applied: -inf where key j > query qidx[i]."""
    if not causal:
        return S
    qidx = np.asarray(qidx).reshape(-1, 1)
    keys = np.arange(S.shape[1]).reshape(1, -1)
    return np.where(keys > qidx, -np.inf, S)


def softmax_rows(S):
    """Row-wise softmax, stabilised by the row maximum (exact in real arithmetic)."""
    S = np.asarray(S, dtype=np.float64)
    m = S.max(axis=-1, keepdims=True)
    E = np.exp(S - m)
    return E / E.sum(axis=-1, keepdims=True)


def attention_forward(Q, K, V, scale, causal=False):
    """Softmax attention forward of one head, O = softmax(scale Q K^T) V.

    The function whose first and second derivatives the abstract is about.
    """
    Q, K, V = _f64(Q, K, V)
    P = softmax_rows(_mask_scores(scale * (Q @ K.T), np.arange(Q.shape[0]), causal))
    return P @ V


def attention_backward(Q, K, V, dO, scale, causal=False):
    """Textbook first backward of one attention head (the pass BoB goes through).

    Abstract: FlashAttention covers the forward and this first backward; BoB
    differentiates through it. Standard form:
      dP = dO V^T,  D = rowsum(dO o O),  dS = P o (dP - D),
      dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
    """
    Q, K, V, dO = _f64(Q, K, V, dO)
    P = softmax_rows(_mask_scores(scale * (Q @ K.T), np.arange(Q.shape[0]), causal))
    O = P @ V
    dP = dO @ V.T
    D = np.sum(dO * O, axis=1, keepdims=True)
    dS = P * (dP - D)
    return scale * (dS @ K), scale * (dS.T @ Q), P.T @ dO


def bob_objective(Q, K, V, dO, gQ, gK, gV, scale, causal=False):
    """Scalar L = <gQ, dQ> + <gK, dK> + <gV, dV> whose gradient BoB returns."""
    dQ, dK, dV = attention_backward(Q, K, V, dO, scale, causal)
    gQ, gK, gV = _f64(gQ, gK, gV)
    return float(np.sum(gQ * dQ) + np.sum(gK * dK) + np.sum(gV * dV))


def _tiles(Q, K, V, dO, gQ, gK, gV, scale, qidx=None, causal=False):
    """All N x N quantities of one head, for the query rows held in Q/dO/gQ.

    Q, dO, gQ may be a block of rows (qidx: their positions in the sequence,
    default 0..); K, V, gK, gV are always all keys. Every quantity below is
    row-local, so a row block gives exact rows.
    """
    if qidx is None:
        qidx = np.arange(Q.shape[0])
    S = _mask_scores(scale * (Q @ K.T), qidx, causal)  # scores
    P = softmax_rows(S)                         # probabilities
    O = P @ V                                   # forward output rows
    D = np.sum(dO * O, axis=1, keepdims=True)   # first-backward row scalar
    dP = dO @ V.T                               # first-backward dP
    dS = P * (dP - D)                           # first-backward dS
    G = scale * (gQ @ K.T + Q @ gK.T)           # adjoint of dS from (gQ, gK)
    H = dO @ gV.T                               # adjoint of P from gV
    c = np.sum(P * G, axis=1, keepdims=True)                 # BoB row scalar 1
    r = (np.sum(dS * G, axis=1, keepdims=True)
         + np.sum(P * H, axis=1, keepdims=True))             # BoB row scalar 2
    A = P * (G - c)                             # dL/d(dP)
    dS2 = dS * (G - c) + P * (H - r)            # dL/dS
    return dict(S=S, P=P, O=O, D=D, dP=dP, dS=dS, G=G, H=H, c=c, r=r, A=A, dS2=dS2)


def bob_head(Q, K, V, dO, gQ, gK, gV, scale, causal=False):
    """Exact BoB of one head: (dL/dQ, dL/dK, dL/dV, dL/ddO), each [N, d].

    Abstract: exact BoB of softmax attention; all outputs are affine in the
    tiles once the two row scalars (c, r) are known. Reverse mode through the
    first backward, one adjoint per node:
      dV = P^T dO         -> dP-bar gets dO gV^T (= H),  ddO-bar gets P gV
      dQ, dK from dS      -> dS-bar = G = scale (gQ K^T + Q gK^T),
                             K-bar gets scale dS^T gQ,  Q-bar gets scale dS gK
      dS = P o (dP - D)   -> dP-bar gets P o G,  D-bar = -c
      D  = rowsum(P o dP) -> dP-bar gets -c P,  so dP-bar = A = P o (G - c)
      dP = dO V^T         -> ddO-bar gets A V,  V-bar = A^T dO
      P  = softmax(S)     -> S-bar = dS2 = dS o (G - c) + P o (H - r)
      S  = scale Q K^T    -> Q-bar gets scale dS2 K,  K-bar gets scale dS2^T Q
    """
    Q, K, V, dO, gQ, gK, gV = _f64(Q, K, V, dO, gQ, gK, gV)
    t = _tiles(Q, K, V, dO, gQ, gK, gV, scale, causal=causal)
    gradQ = scale * (t["dS2"] @ K + t["dS"] @ gK)
    gradK = scale * (t["dS2"].T @ Q + t["dS"].T @ gQ)
    gradV = t["A"].T @ dO
    graddO = t["A"] @ V + t["P"] @ gV
    return gradQ, gradK, gradV, graddO


def bob(Q, K, V, dO, gQ, gK, gV, scale, causal=False):
    """Batched BoB over leading dims [..., N, d]; each (b, h) slice independently."""
    Q, K, V, dO, gQ, gK, gV = _f64(Q, K, V, dO, gQ, gK, gV)
    lead = Q.shape[:-2]
    outs = [np.empty_like(Q), np.empty_like(K), np.empty_like(V), np.empty_like(dO)]
    for idx in np.ndindex(*lead):
        res = bob_head(Q[idx], K[idx], V[idx], dO[idx], gQ[idx], gK[idx], gV[idx], scale, causal)
        for o, x in zip(outs, res):
            o[idx] = x
    return tuple(outs)


def row_stats_head(Q, K, V, dO, gQ, gK, gV, scale, causal=False):
    """Per-row scalars of one head by their direct definitions: (LSE, D, c, r), each [N].

    LSE is the log of the softmax normaliser of scale Q K^T; D is the
    first-backward row scalar; c and r are the two BoB row scalars.
    """
    Q, K, V, dO, gQ, gK, gV = _f64(Q, K, V, dO, gQ, gK, gV)
    t = _tiles(Q, K, V, dO, gQ, gK, gV, scale, causal=causal)
    S = t["S"]
    m = S.max(axis=1)
    lse = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    return lse, t["D"][:, 0], t["c"][:, 0], t["r"][:, 0]


def row_stats_closed_forms_head(Q, K, V, dO, gQ, gK, gV, scale, causal=False):
    """(D, c, r) of one head through d-vector contractions instead of N x N rowsums.

    D = dO . (P V),   c = scale (gQ . (P K) + Q . (P gK)),
    r = gQ . dQ + scale Q . (dS gK) + dO . (P gV).
    A second route to the row scalars, used to cross-check the first.
    """
    Q, K, V, dO, gQ, gK, gV = _f64(Q, K, V, dO, gQ, gK, gV)
    P = softmax_rows(_mask_scores(scale * (Q @ K.T), np.arange(Q.shape[0]), causal))
    D = np.sum(dO * (P @ V), axis=1)
    c = scale * (np.sum(gQ * (P @ K), axis=1) + np.sum(Q * (P @ gK), axis=1))
    dS = P * (dO @ V.T - D[:, None])
    dQ = scale * (dS @ K)
    r = np.sum(gQ * dQ, axis=1) + scale * np.sum(Q * (dS @ gK), axis=1) \
        + np.sum(dO * (P @ gV), axis=1)
    return D, c, r


def row_stats_online_head(Q, K, V, dO, gQ, gK, gV, scale, block, causal=False):
    """(LSE, D, c, r) of one head in one sweep over key blocks (online softmax).

    The row scalars only need running sums weighted by exp(S - m): l, and the
    weighted sums of dP, G, dP o G and H, all rescaled when the running max m
    grows (online normaliser of the cited softmax work). Finalise:
      LSE = m + ln l,  D = a_D / l,  c = a_c / l,  r = a_e / l - D c + a_h / l.
    """
    Q, K, V, dO, gQ, gK, gV = _f64(Q, K, V, dO, gQ, gK, gV)
    N = Q.shape[0]
    m = np.full(N, -np.inf)
    l = np.zeros(N)
    aD = np.zeros(N)
    ac = np.zeros(N)
    ae = np.zeros(N)
    ah = np.zeros(N)
    for j0 in range(0, K.shape[0], block):
        j1 = min(j0 + block, K.shape[0])
        S = scale * (Q @ K[j0:j1].T)
        if causal:  # key j0 + k is masked for query i when j0 + k > i
            S = np.where(np.arange(j0, j1)[None, :] > np.arange(N)[:, None], -np.inf, S)
        G = scale * (gQ @ K[j0:j1].T + Q @ gK[j0:j1].T)
        dP = dO @ V[j0:j1].T
        H = dO @ gV[j0:j1].T
        m_new = np.maximum(m, S.max(axis=1))
        # (a block masked for a whole row leaves m at -inf only while every
        # earlier block was masked too, which never happens: key 0 is always
        # visible)
        alpha = np.exp(m - m_new)
        Pt = np.exp(S - m_new[:, None])
        l = alpha * l + Pt.sum(axis=1)
        aD = alpha * aD + np.sum(Pt * dP, axis=1)
        ac = alpha * ac + np.sum(Pt * G, axis=1)
        ae = alpha * ae + np.sum(Pt * dP * G, axis=1)
        ah = alpha * ah + np.sum(Pt * H, axis=1)
        m = m_new
    D = aD / l
    c = ac / l
    r = ae / l - D * c + ah / l
    return m + np.log(l), D, c, r


def bob_rows_head(Q, K, V, dO, gQ, gK, gV, scale, rows, causal=False):
    """gradQ and graddO of one head for the query rows `rows` only (exact).

    Both are row-local: every N x N quantity of a query row depends on that
    row and on all keys, so the rows' values equal the full computation's.
    """
    Q, K, V, dO, gQ, gK, gV = _f64(Q, K, V, dO, gQ, gK, gV)
    rows = np.asarray(rows)
    t = _tiles(Q[rows], K, V, dO[rows], gQ[rows], gK, gV, scale, qidx=rows, causal=causal)
    gradQ = scale * (t["dS2"] @ K + t["dS"] @ gK)
    graddO = t["A"] @ V + t["P"] @ gV
    return gradQ, graddO


def bob_blocked_head(Q, K, V, dO, gQ, gK, gV, scale, block=1024, causal=False):
    """bob_head computed over blocks of query rows to bound host memory.

    Rows of gradQ and graddO are final per block; gradK and gradV are sums of
    per-block contributions over all query rows.
    """
    Q, K, V, dO, gQ, gK, gV = _f64(Q, K, V, dO, gQ, gK, gV)
    N = Q.shape[0]
    gradQ = np.empty_like(Q)
    graddO = np.empty_like(dO)
    gradK = np.zeros_like(K)
    gradV = np.zeros_like(V)
    for i0 in range(0, N, block):
        I = slice(i0, min(i0 + block, N))
        t = _tiles(Q[I], K, V, dO[I], gQ[I], gK, gV, scale, qidx=np.arange(N)[I], causal=causal)
        gradQ[I] = scale * (t["dS2"] @ K + t["dS"] @ gK)
        graddO[I] = t["A"] @ V + t["P"] @ gV
        gradK += scale * (t["dS2"].T @ Q[I] + t["dS"].T @ gQ[I])
        gradV += t["A"].T @ dO[I]
    return gradQ, gradK, gradV, graddO


def bob_blocked(Q, K, V, dO, gQ, gK, gV, scale, block=1024, causal=False):
    """Batched row-blocked BoB over leading dims [..., N, d]."""
    Q, K, V, dO, gQ, gK, gV = _f64(Q, K, V, dO, gQ, gK, gV)
    lead = Q.shape[:-2]
    outs = [np.empty_like(Q), np.empty_like(K), np.empty_like(V), np.empty_like(dO)]
    for idx in np.ndindex(*lead):
        res = bob_blocked_head(Q[idx], K[idx], V[idx], dO[idx], gQ[idx], gK[idx],
                               gV[idx], scale, block, causal)
        for o, x in zip(outs, res):
            o[idx] = x
    return tuple(outs)


def bob_gqa(Q, K, V, dO, gQ, gK, gV, scale, causal=False, block=None):
    """Batched BoB with grouped key/value heads (GQA / MQA).

    Q, dO, gQ are [B, H, N, d]; K, V, gK, gV are [B, Hkv, N, d] with H a
    multiple of Hkv, and query head h uses key/value head h // (H / Hkv) (a
    reading beyond the pages). The first backward of such attention gives the
    shared K and V the sum of their per-head gradients, so L = <gQ, dQ> +
    <gK, dK> + <gV, dV> is the multi-head objective with K, V, gK, gV repeated
    over each group: gradQ, graddO are per query head, gradK, gradV are the
    sums over the group's query heads. `block` selects the row-blocked form.
    """
    Q, K, V, dO, gQ, gK, gV = _f64(Q, K, V, dO, gQ, gK, gV)
    B, H = Q.shape[:2]
    Hkv = K.shape[1]
    if H % Hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    G = H // Hkv
    gradQ = np.empty_like(Q)
    graddO = np.empty_like(dO)
    gradK = np.zeros_like(K)
    gradV = np.zeros_like(V)
    for b in range(B):
        for h in range(H):
            j = h // G
            args = (Q[b, h], K[b, j], V[b, j], dO[b, h], gQ[b, h], gK[b, j], gV[b, j], scale)
            if block is None:
                gq, gk, gv, gdo = bob_head(*args, causal=causal)
            else:
                gq, gk, gv, gdo = bob_blocked_head(*args, block=block, causal=causal)
            gradQ[b, h] = gq
            graddO[b, h] = gdo
            gradK[b, j] += gk
            gradV[b, j] += gv
    return gradQ, gradK, gradV, graddO


def attention_backward_batched(Q, K, V, dO, scale, causal=False):
    """First backward (dQ, dK, dV) over [B, H, N, d] queries and [B, Hkv, N, d]
    keys/values (Hkv divides H; query head h uses key/value head h // (H/Hkv),
    and the shared heads' dK, dV sum over the group)."""
    Q, K, V, dO = _f64(Q, K, V, dO)
    B, H = Q.shape[:2]
    G = H // K.shape[1]
    dQ = np.empty_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for b in range(B):
        for h in range(H):
            j = h // G
            q, k, v = attention_backward(Q[b, h], K[b, j], V[b, j], dO[b, h], scale, causal)
            dQ[b, h] = q
            dK[b, j] += k
            dV[b, j] += v
    return dQ, dK, dV


def attention_backward_rows_head(Q, K, V, dO, scale, rows, causal=False):
    """First-backward dQ of one head for the query rows `rows` only (exact).

    dQ_i = scale sum_j dS_ij K_j needs, besides row i of Q and dO, only that
    row's softmax and D_i = dO_i . O_i, so the rows' values equal those of
    the full first backward (same formulas as attention_backward).
    """
    Q, K, V, dO = _f64(Q, K, V, dO)
    rows = np.asarray(rows)
    P = softmax_rows(_mask_scores(scale * (Q[rows] @ K.T), rows, causal))
    dOr = dO[rows]
    D = np.sum(dOr * (P @ V), axis=1, keepdims=True)
    dS = P * (dOr @ V.T - D)
    return scale * (dS @ K)
