"""Brute-force Python ``decimal`` versions of the oracle's definitions (tiny inputs).

TEST INFRASTRUCTURE ONLY; used to pin the float64 oracle, never by the product.

Pure-Python loops at 50 significant digits, sharing no code with
``flare_ref``.  They restate the same definitions from the pages:
"FLARE++: Low-rank attention with dynamic attention routing" (appendix on
context parallelism: eq. 18, the local-shard (O_r, L_r) states with the empty
rule, the merge, the FLARE decode, the backward with global statistics) and
"Ring vs. Tree Attention" (the (m, l) merge).
"""
from __future__ import annotations

from decimal import Decimal, getcontext

getcontext().prec = 50

NEG = None  # stands for -inf in this module


def D_(x) -> Decimal:
    return Decimal(float(x))   # exact binary value of the float


def dot(a, b):
    s = Decimal(0)
    for x, y in zip(a, b):
        s += x * y
    return s


def softmax_attend(scores, values):
    """scores: list of Decimals (valid columns only); values: list of rows.

    Returns (out row-vector, lse) or (zeros, NEG) with no column.
    """
    if len(scores) == 0:
        return [Decimal(0)] * (len(values[0]) if values else 0), NEG
    mx = max(scores)
    w = [(s - mx).exp() for s in scores]
    l = sum(w, Decimal(0))
    D = len(values[0])
    out = []
    for d in range(D):
        acc = Decimal(0)
        for wi, v in zip(w, values):
            acc += wi * v[d]
        out.append(acc / l)
    return out, mx + l.ln()


def encode(q, k, v, valid, offsets, scale):
    """q: M rows, k/v: N rows (floats); returns (parts, (Z, L)); parts[r] = (O rows, L list)."""
    s = D_(scale)
    Q = [[D_(x) for x in row] for row in q]
    K = [[D_(x) for x in row] for row in k]
    V = [[D_(x) for x in row] for row in v]
    D = len(V[0])

    def run(cols):
        Os, Ls = [], []
        for qm in Q:
            sc = [s * dot(qm, K[n]) for n in cols]
            o, l = softmax_attend(sc, [V[n] for n in cols])
            if not cols:
                o = [Decimal(0)] * D
            Os.append(o)
            Ls.append(l)
        return Os, Ls

    parts = []
    for r in range(len(offsets) - 1):
        cols = [n for n in range(offsets[r], offsets[r + 1]) if valid[n]]
        parts.append(run(cols))
    cols = [n for n in range(len(K)) if valid[n]]
    return parts, run(cols)


def merge_oneshot(parts):
    """parts: list of (O rows, L list) -> (Z rows, L list), via L_max, a_r, a, U."""
    R = len(parts)
    M = len(parts[0][1])
    D = len(parts[0][0][0])
    Z, L = [], []
    for m in range(M):
        Ls = [parts[r][1][m] for r in range(R)]
        fin = [x for x in Ls if x is not NEG]
        if not fin:
            Z.append([Decimal(0)] * D)
            L.append(NEG)
            continue
        Lmax = max(fin)
        a_r = [Decimal(0) if x is NEG else (x - Lmax).exp() for x in Ls]
        a = sum(a_r, Decimal(0))
        U = [sum((a_r[r] * parts[r][0][m][d] for r in range(R)), Decimal(0)) for d in range(D)]
        Z.append([u / a for u in U])
        L.append(Lmax + a.ln())
    return Z, L


def merge_ml(pairs):
    """Ring-order fold of (m, l) pairs with m = max(m1, m2), l = l1 e^(m1-m) + l2 e^(m2-m)."""
    m, l = D_(pairs[0][0]), D_(pairs[0][1])
    for m2, l2 in pairs[1:]:
        m2, l2 = D_(m2), D_(l2)
        mm = max(m, m2)
        l = l * (m - mm).exp() + l2 * (m2 - mm).exp()
        m = mm
    return m, l


def decode(xq, klat, z, scale):
    s = D_(scale)
    X = [[D_(x) for x in row] for row in xq]
    Kl = [[D_(x) for x in row] for row in klat]
    Zr = [[D_(x) for x in row] for row in z]
    Y = []
    for xn in X:
        sc = [s * dot(xn, km) for km in Kl]
        y, _ = softmax_attend(sc, Zr)
        Y.append(y)
    return Y


def encode_bwd(q, k, v, valid, scale, dZ):
    """Gradients of <dZ, Z> with Z = softmax(s q k^T) v over the valid columns.

    Written from the chain rule directly (softmax Jacobian), not from the
    P / c / dS factorisation: dZ[m] . dZ_m/dS[m,n] = P[m,n] (dZ[m].v[n] - dZ[m].Z[m]).
    """
    s = D_(scale)
    Q = [[D_(x) for x in row] for row in q]
    K = [[D_(x) for x in row] for row in k]
    V = [[D_(x) for x in row] for row in v]
    G = [[D_(x) for x in row] for row in dZ]
    M, D, N = len(Q), len(Q[0]), len(K)
    cols = [n for n in range(N) if valid[n]]
    dq = [[Decimal(0)] * D for _ in range(M)]
    dk = [[Decimal(0)] * D for _ in range(N)]
    dv = [[Decimal(0)] * D for _ in range(N)]
    for m in range(M):
        sc = [s * dot(Q[m], K[n]) for n in cols]
        if not sc:
            continue
        mx = max(sc)
        w = [(x - mx).exp() for x in sc]
        tot = sum(w, Decimal(0))
        p = [x / tot for x in w]
        z = [sum((p[i] * V[n][d] for i, n in enumerate(cols)), Decimal(0)) for d in range(D)]
        gz = dot(G[m], z)
        for i, n in enumerate(cols):
            g_s = p[i] * (dot(G[m], V[n]) - gz)       # d<dZ,Z>/dS[m,n]
            for d in range(D):
                dv[n][d] += p[i] * G[m][d]
                dk[n][d] += s * g_s * Q[m][d]
                dq[m][d] += s * g_s * K[n][d]
    return dq, dk, dv
