"""Plain, slow, obviously correct CPU oracle for the split-KV / FLARE softmax path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code with the HIP library.

Everything is float64 numpy and materialises the full score matrix of each
(batch, head) slice.  Inputs are widened exactly from the bits the GPU
receives (bfloat16 -> float32 -> float64 is exact), and the scale is the same
float32 value of D^-1/2 that the kernels take.

Sources (page title, then the part of the page):

* "FLARE++: Low-rank attention with dynamic attention routing", appendix on
  context parallelism:
  - eq. 18, the encoder result Z = softmax(s Q K^T) V over the whole token
    sequence, with s = D^-1/2 and padding excluded by the key mask;
  - the local-shard equations that follow it: each shard r returns its own
    normalised output O_r and log-normaliser L_r, with (O_r, L_r) = (0, -inf)
    for an attention row that has no valid key in the shard;
  - the global log-normaliser L = log sum_r exp L_r, the shard mass
    alpha_r = exp(L_r - L), and eq. 23, Z = sum_r alpha_r O_r;
  - the max-stabilised merge paragraph (L_max, a_r = exp(L_r - L_max),
    a = sum a_r, U = sum a_r O_r);
  - the FLARE paragraph (decode of every token against the replicated latents)
    and the FLARE++ paragraph (two encoders then one decode);
  - the backward paragraph: P_r = exp(S_r - L) with the global L, the row term
    c = rowsum(dZ * Z), and the local gradients of K_r, V_r plus the summed
    query gradient.
* "Ring vs. Tree Attention": the online-softmax merge of (m, l) states with
  its separately rescaled output accumulator, the ring (left fold) and the
  balanced tree schedules, and the proposition that the merge is a
  commutative semigroup.

Readings taken where the pages are silent (display equations were lost in
extraction) are listed in the repository's design notes; the main ones are:
the decode's token-side query is the token's own key row and its keys/values
are the latent queries and Z; the same scale s is used everywhere; log is the
natural logarithm; a row with no valid key anywhere returns (0, -inf).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf


# ----------------------------------------------------------------------------
# input handling
# ----------------------------------------------------------------------------
def f64(x) -> np.ndarray:
    """Exact widening of a torch tensor (any float dtype) or array to float64."""
    if hasattr(x, "detach"):
        import torch
        t = x.detach().cpu()
        if t.dtype in (torch.bfloat16, torch.float16):
            t = t.to(torch.float32)
        return t.numpy().astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def u8(x) -> np.ndarray:
    if hasattr(x, "detach"):
        return x.detach().cpu().numpy().astype(np.uint8)
    return np.asarray(x, dtype=np.uint8)


def _q_slice(Q: np.ndarray, b: int, h: int) -> np.ndarray:
    """Q is either replicated [H, M, D] or per batch [B, H, M, D]."""
    return Q[h] if Q.ndim == 3 else Q[b, h]


# ----------------------------------------------------------------------------
# the plain definition on one set of columns (eq. 18 / the local-shard form)
# ----------------------------------------------------------------------------
def attend(S: np.ndarray, V: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax over the columns of S applied to V, plus the row log-sum-exp.

    S: [M, n] scores of the columns that take part (all of them valid);
    V: [n, D].  Returns O [M, D] and L [M].  With no column, O = 0 and
    L = -inf (the empty-row rule of the local-shard paragraph).
    """
    M = S.shape[0]
    D = V.shape[1]
    if S.shape[1] == 0:
        return np.zeros((M, D)), np.full(M, NEG_INF)
    mx = S.max(axis=1)
    w = np.exp(S - mx[:, None])
    l = w.sum(axis=1)
    O = (w @ V) / l[:, None]
    L = mx + np.log(l)
    return O, L


def slice_scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = s * q k^T for one (batch, head) slice: [M, n]."""
    return float(scale) * (q @ k.T)


# ----------------------------------------------------------------------------
# encoder: per-partition states and the global result
# ----------------------------------------------------------------------------
def encode_slice(q, k, v, valid, offsets: Sequence[int], scale: float):
    """One (b, h) slice: ([O_r], [L_r]) for every partition and the global (Z, L)."""
    S = slice_scores(q, k, scale)
    valid = np.asarray(valid).astype(bool)
    O_parts, L_parts = [], []
    for r in range(len(offsets) - 1):
        lo, hi = int(offsets[r]), int(offsets[r + 1])
        cols = lo + np.nonzero(valid[lo:hi])[0]
        O, L = attend(S[:, cols], v[cols])
        O_parts.append(O)
        L_parts.append(L)
    cols = np.nonzero(valid)[0]
    Z, L = attend(S[:, cols], v[cols])
    return O_parts, L_parts, Z, L


def encode_ref(Q, K, V, offsets: Sequence[int], mask=None, scale: float = None,
               slices: Optional[List[Tuple[int, int]]] = None) -> Dict[str, np.ndarray]:
    """Encoder over all (b, h) slices, or only the listed ones.

    Q: [H, M, D] (replicated over the batch) or [B, H, M, D]; K, V: [B, H, N, D];
    mask: [B, N] (nonzero = valid key) or None.
    Returns O_part [R, B, H, M, D], L_part [R, B, H, M], Z [B, H, M, D], L [B, H, M]
    (slices that were not asked for are left as NaN).
    """
    Q, K, V = f64(Q), f64(K), f64(V)
    B, H, N, D = K.shape
    M = Q.shape[-2]
    R = len(offsets) - 1
    mk = np.ones((B, N), dtype=np.uint8) if mask is None else u8(mask)
    if scale is None:
        scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    out = {
        "O_part": np.full((R, B, H, M, D), np.nan), "L_part": np.full((R, B, H, M), np.nan),
        "Z": np.full((B, H, M, D), np.nan), "L": np.full((B, H, M), np.nan),
    }
    todo = slices if slices is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        Op, Lp, Z, L = encode_slice(_q_slice(Q, b, h), K[b, h], V[b, h], mk[b], offsets, scale)
        for r in range(R):
            out["O_part"][r, b, h] = Op[r]
            out["L_part"][r, b, h] = Lp[r]
        out["Z"][b, h] = Z
        out["L"][b, h] = L
    return out


# ----------------------------------------------------------------------------
# merges of partition states
# ----------------------------------------------------------------------------
def merge_oneshot(O_part: np.ndarray, L_part: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """The max-stabilised cross-shard merge of the FLARE++ appendix.

    L_max = max_r L_r, a_r = exp(L_r - L_max), a = sum_r a_r,
    U = sum_r a_r O_r (a_r broadcast over D), Z = U / a, L = L_max + log a.
    Rows where every L_r is -inf give Z = 0, L = -inf.
    """
    O_part = np.asarray(O_part, dtype=np.float64)
    L_part = np.asarray(L_part, dtype=np.float64)
    L_max = L_part.max(axis=0)
    empty = np.isneginf(L_max)
    safe = np.where(empty, 0.0, L_max)
    a_r = np.where(np.isneginf(L_part), 0.0, np.exp(L_part - safe[None]))
    a = a_r.sum(axis=0)
    U = (a_r[..., None] * O_part).sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        Z = np.where(empty[..., None], 0.0, U / np.where(empty, 1.0, a)[..., None])
        L = np.where(empty, NEG_INF, safe + np.log(np.where(empty, 1.0, a)))
    return Z, L


# (m, l, acc) online-softmax states, as on the ring-vs-tree page
def state_of(O_r: np.ndarray, L_r: np.ndarray):
    """A partition's (O_r, L_r) as an (m, l, acc) state: m = L_r, l = 1, acc = O_r.

    An empty partition (L_r = -inf) is the identity state (-inf, 0, 0).
    """
    O_r = np.asarray(O_r, dtype=np.float64)
    L_r = np.asarray(L_r, dtype=np.float64)
    e = np.isneginf(L_r)
    return L_r.copy(), np.where(e, 0.0, 1.0), np.where(e[..., None], 0.0, O_r)


def merge_states(s1, s2):
    """m = max(m1, m2); l = l1 e^(m1-m) + l2 e^(m2-m); acc rescaled like l."""
    m1, l1, a1 = s1
    m2, l2, a2 = s2
    m = np.maximum(m1, m2)
    both_empty = np.isneginf(m)
    ms = np.where(both_empty, 0.0, m)
    f1 = np.where(np.isneginf(m1), 0.0, np.exp(m1 - ms))
    f2 = np.where(np.isneginf(m2), 0.0, np.exp(m2 - ms))
    return m, l1 * f1 + l2 * f2, a1 * f1[..., None] + a2 * f2[..., None]


def finish_state(s):
    """Z = acc / l and L = m + log l; an empty state gives (0, -inf)."""
    m, l, a = s
    empty = l == 0
    with np.errstate(invalid="ignore", divide="ignore"):
        Z = np.where(empty[..., None], 0.0, a / np.where(empty, 1.0, l)[..., None])
        L = np.where(empty, NEG_INF, m + np.log(np.where(empty, 1.0, l)))
    return Z, L


def fold_tree(states: List):
    """Balanced binary tree: round k merges i and i + 2^k for i = 0 mod 2^(k+1).

    A survivor without a partner in a round passes through unchanged.
    """
    cur = list(states)
    R = len(cur)
    step = 1
    while step < R:
        for i in range(0, R, 2 * step):
            if i + step < R:
                cur[i] = merge_states(cur[i], cur[i + step])
        step *= 2
    return cur[0]


def fold_left(states: List):
    """The ring order: ((s0 . s1) . s2) . ..."""
    acc = states[0]
    for s in states[1:]:
        acc = merge_states(acc, s)
    return acc


def merge_tree(O_part, L_part):
    return finish_state(fold_tree([state_of(O_part[r], L_part[r]) for r in range(len(L_part))]))


def merge_leftfold(O_part, L_part):
    return finish_state(fold_left([state_of(O_part[r], L_part[r]) for r in range(len(L_part))]))


# ----------------------------------------------------------------------------
# decode (FLARE paragraph) and the FLARE++ chain
# ----------------------------------------------------------------------------
def decode_slice(xq, klat, z, scale: float) -> np.ndarray:
    """Every token row of xq attends over the M latent rows: softmax(s xq klat^T) z."""
    T = float(scale) * (xq @ klat.T)              # [n, M]
    mx = T.max(axis=1)
    w = np.exp(T - mx[:, None])
    return (w @ z) / w.sum(axis=1)[:, None]


def decode_ref(Xq, Klat, Z, scale: float, token_mask=None,
               slices: Optional[List[Tuple[int, int]]] = None) -> np.ndarray:
    """Y [B, H, N, D]; Klat is [H, M, D] or [B, H, M, D]; masked token rows give Y = 0."""
    Xq, Klat, Z = f64(Xq), f64(Klat), f64(Z)
    B, H, N, D = Xq.shape
    Y = np.full((B, H, N, D), np.nan)
    mk = None if token_mask is None else u8(token_mask).astype(bool)
    todo = slices if slices is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        y = decode_slice(Xq[b, h], _q_slice(Klat, b, h), Z[b, h], scale)
        if mk is not None:
            y[~mk[b]] = 0.0
        Y[b, h] = y
    return Y


def bf16_round(x: np.ndarray) -> np.ndarray:
    """x rounded to bfloat16 (to float32, then to nearest even bfloat16) and widened back.

    The kernels hold Q(X) in float32 and round that to bfloat16; the detour
    through float32 reproduces that.  NaN stays NaN (it marks a (batch, head)
    slice that was not computed when only some slices are)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(torch.bfloat16).to(
        torch.float64).numpy()


def flarepp_ref(Qt, Kt, Vt, K, V, offsets, scale: float, round_qx_bf16: bool = False,
                slices: Optional[List[Tuple[int, int]]] = None) -> Dict[str, np.ndarray]:
    """FLARE++ forward: Q(X) = Enc(Qt, Kt, Vt); Z = Enc(Q(X), K, V); Y = Dec(K, Q(X), Z).

    With ``round_qx_bf16`` the dynamic queries are rounded to bfloat16 before
    the second encoder and the decode (the precision the kernels consume them
    in); by default the oracle keeps them in float64.
    """
    e1 = encode_ref(Qt, Kt, Vt, offsets, None, scale, slices=slices)
    QX = e1["Z"]
    QXu = bf16_round(QX) if round_qx_bf16 else QX
    e2 = encode_ref(QXu, K, V, offsets, None, scale, slices=slices)
    Y = decode_ref(K, QXu, e2["Z"], scale, slices=slices)
    return {"QX": QX, "QX_L": e1["L"], "QX_O_part": e1["O_part"], "QX_L_part": e1["L_part"],
            "Z": e2["Z"], "L": e2["L"], "O_part": e2["O_part"], "L_part": e2["L_part"], "Y": Y}


# ----------------------------------------------------------------------------
# encoder backward with the global statistics (backward paragraph)
# ----------------------------------------------------------------------------
def encode_bwd_slice(q, k, v, valid, scale: float, Z, L, dZ):
    """dq [M, D], dk [n, D], dv [n, D] of <dZ, Z(q, k, v)> using the global Z and L.

    P = exp(S - L) on the valid columns (0 elsewhere), c = rowsum(dZ * Z),
    dP = dZ v^T, dS = P * (dP - c), dv = P^T dZ, dk = s dS^T q, dq = s dS k.
    Rows whose L is -inf have P = 0.
    """
    valid = np.asarray(valid).astype(bool)
    N, D = k.shape
    cols = np.nonzero(valid)[0]
    S = slice_scores(q, k[cols], scale)
    Ls = np.where(np.isneginf(L), np.inf, L)
    P = np.exp(S - Ls[:, None])
    c = (dZ * Z).sum(axis=1)
    dP = dZ @ v[cols].T
    dS = P * (dP - c[:, None])
    dk = np.zeros((N, D))
    dv = np.zeros((N, D))
    dv[cols] = P.T @ dZ
    dk[cols] = float(scale) * (dS.T @ q)
    dq = float(scale) * (dS @ k[cols])
    return dq, dk, dv


def encode_bwd_ref(Q, K, V, mask, scale: float, Z, L, dZ,
                   slices: Optional[List[Tuple[int, int]]] = None) -> Dict[str, np.ndarray]:
    """dQ [B, H, M, D] (one per batch even when Q is replicated), dK, dV [B, H, N, D]."""
    Q, K, V, Z, L, dZ = f64(Q), f64(K), f64(V), f64(Z), f64(L), f64(dZ)
    B, H, N, D = K.shape
    M = Q.shape[-2]
    mk = np.ones((B, N), dtype=np.uint8) if mask is None else u8(mask)
    out = {"dQ": np.full((B, H, M, D), np.nan), "dK": np.full((B, H, N, D), np.nan),
           "dV": np.full((B, H, N, D), np.nan)}
    todo = slices if slices is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        dq, dk, dv = encode_bwd_slice(_q_slice(Q, b, h), K[b, h], V[b, h], mk[b], scale,
                                      Z[b, h], L[b, h], dZ[b, h])
        out["dQ"][b, h], out["dK"][b, h], out["dV"][b, h] = dq, dk, dv
    return out


def encode_bwd_local_slice(q, k, v, valid, offsets, scale: float, dZ):
    """Negative control: each partition differentiated as its own attention.

    Uses the shard's own L_r and O_r (and c_r = rowsum(dZ * O_r)) in place of
    the global statistics.  The backward paragraph says this omits the
    between-shard term, so its gradients must differ from encode_bwd_slice.
    """
    Op, Lp, _, _ = encode_slice(q, k, v, valid, offsets, scale)
    M, D = q.shape
    dq = np.zeros((M, D))
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r in range(len(offsets) - 1):
        lo, hi = int(offsets[r]), int(offsets[r + 1])
        sub = np.zeros(k.shape[0], dtype=bool)
        sub[lo:hi] = np.asarray(valid[lo:hi]).astype(bool)
        a, b_, c_ = encode_bwd_slice(q, k, v, sub, scale, Op[r], Lp[r], dZ)
        dq += a
        dk += b_
        dv += c_
    return dq, dk, dv


# ----------------------------------------------------------------------------
# decode backward and the FLARE++ backward chain (FLARE++ backward paragraph:
# the decoder's contributions to the replicated latents are summed, the
# decoder's query-gradient is added to the physical-value encoder's, and the
# sum is propagated through the query-synthesis encoder with that invocation's
# own saved output and log-normaliser)
# ----------------------------------------------------------------------------
def decode_bwd_slice(xq, klat, z, scale: float, dy, valid=None):
    """Gradients of <dY, Y> for Y = softmax(s xq klat^T) z, one (batch, head) slice.

    A = softmax over the M latents of T = s xq klat^T; dA = dy z^T; the row
    term delta = rowsum(A * dA) (= rowsum(dy * y)); dT = A * (dA - delta);
    dxq = s dT klat, dklat = s dT^T xq, dz = A^T dy.  Masked tokens (their Y is
    0 by definition) take no part: zero dxq rows, no contribution to dklat, dz.
    """
    n, D = xq.shape
    keep = np.ones(n, dtype=bool) if valid is None else np.asarray(valid).astype(bool)
    T = float(scale) * (xq @ klat.T)                      # [n, M]
    A = np.exp(T - T.max(axis=1, keepdims=True))
    A /= A.sum(axis=1, keepdims=True)
    dyk = np.where(keep[:, None], dy, 0.0)
    dA = dyk @ z.T
    delta = (A * dA).sum(axis=1)
    dT = A * (dA - delta[:, None])
    dxq = float(scale) * (dT @ klat)
    dklat = float(scale) * (dT.T @ xq)
    dz = A.T @ dyk
    return dxq, dklat, dz


def decode_bwd_ref(Xq, Klat, Z, scale: float, dY, token_mask=None,
                   slices: Optional[List[Tuple[int, int]]] = None) -> Dict[str, np.ndarray]:
    """dXq [B, H, N, D], dKlat [B, H, M, D] (one per batch even when Klat is replicated),
    dZ [B, H, M, D] of <dY, decode(Xq, Klat, Z)>."""
    Xq, Klat, Z, dY = f64(Xq), f64(Klat), f64(Z), f64(dY)
    B, H, N, D = Xq.shape
    M = Klat.shape[-2]
    mk = np.ones((B, N), dtype=bool) if token_mask is None else u8(token_mask).astype(bool)
    out = {"dXq": np.full((B, H, N, D), np.nan), "dKlat": np.full((B, H, M, D), np.nan),
           "dZ": np.full((B, H, M, D), np.nan)}
    todo = slices if slices is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        a, k, z = decode_bwd_slice(Xq[b, h], _q_slice(Klat, b, h), Z[b, h], scale, dY[b, h], mk[b])
        out["dXq"][b, h], out["dKlat"][b, h], out["dZ"][b, h] = a, k, z
    return out


def flarepp_shared_bwd_ref(Qt, K, V, offsets, scale: float, dY, round_qx_bf16: bool = False,
                           slices: Optional[List[Tuple[int, int]]] = None) -> Dict[str, np.ndarray]:
    """Gradients of <dY, Y> for the shared-projection variant of FLARE++ ("FLARE++",
    paragraph on the cost of the two extra projections: the query-synthesis
    encoder's keys and values tied to K and V).  K and V then enter all three
    attention calls, so their gradients are the sums of the three calls'
    contributions: dK = dK_dec + dK_enc2 + dK_enc1, dV = dV_enc2 + dV_enc1."""
    g = flarepp_bwd_ref(Qt, K, V, K, V, offsets, scale, dY, round_qx_bf16=round_qx_bf16, slices=slices)
    return {"dQt": g["dQt"], "dK": g["dK"] + g["dKt"], "dV": g["dV"] + g["dVt"], "dQX": g["dQX"],
            "forward": g["forward"]}


def flarepp_bwd_ref(Qt, Kt, Vt, K, V, offsets, scale: float, dY, round_qx_bf16: bool = False,
                    slices: Optional[List[Tuple[int, int]]] = None) -> Dict[str, np.ndarray]:
    """Gradients of <dY, Y> for the FLARE++ chain of flarepp_ref.

    decoder: (dK_dec, dQX_dec, dZ2) = decode backward at (K, Q(X), Z2);
    physical-value encoder: (dQX_enc, dK_enc, dV) = encoder backward at (Q(X), K, V)
    with its own (Z2, L2) and dZ2;  dQX = dQX_dec + dQX_enc;
    query-synthesis encoder: (dQt, dKt, dVt) = encoder backward at (Qt, Kt, Vt) with
    its own (Q(X), L1) and dQX.  dK = dK_dec + dK_enc.  With ``round_qx_bf16``
    the second encoder and the decoder see Q(X) rounded to bfloat16 (as the
    kernels do) and its gradient passes the rounding unchanged.
    """
    f = flarepp_ref(Qt, Kt, Vt, K, V, offsets, scale, round_qx_bf16=round_qx_bf16, slices=slices)
    QX = f["QX"]
    QXu = bf16_round(QX) if round_qx_bf16 else QX
    d = decode_bwd_ref(K, QXu, f["Z"], scale, dY, slices=slices)
    g2 = encode_bwd_ref(QXu, K, V, None, scale, f["Z"], f["L"], d["dZ"], slices=slices)
    dQX = d["dKlat"] + g2["dQ"]
    g1 = encode_bwd_ref(Qt, Kt, Vt, None, scale, QX, f["QX_L"], dQX, slices=slices)
    return {"dQt": g1["dQ"], "dKt": g1["dK"], "dVt": g1["dV"], "dK": d["dXq"] + g2["dK"], "dV": g2["dV"],
            "dQX": dQX, "dQX_dec": d["dKlat"], "dZ2": d["dZ"], "forward": f}
