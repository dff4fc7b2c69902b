"""Pins of the CPU oracle against what the pages and the mathematics fix (CPU only).

Each test names the part of the pages it follows:
* "FLARE++: Low-rank attention with dynamic attention routing" (appendix on
  context parallelism): eq. 18, the local-shard states and the empty rule,
  eq. 23, the max-stabilised merge, the FLARE / FLARE++ paragraphs, the
  backward paragraph (global statistics, the row term c, the warning that a
  local backward misses the between-shard term), and the remark that token
  order carries no meaning.
* "Ring vs. Tree Attention": the (m, l) merge, the commutative-semigroup
  proposition, the failure mode (double counting), and the core exercise.
"""
import json
import math
import os
import random

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import brute
from oracle import flare_ref as ref

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng0 = np.random.default_rng(1234)


def _rand_problem(rng, B=2, H=2, M=5, N=40, D=8, R=4, masked=True, empty_part=True, qscale=1.0):
    Q = rng.standard_normal((H, M, D)) * qscale
    K = rng.standard_normal((B, H, N, D))
    V = rng.standard_normal((B, H, N, D))
    cuts = sorted(rng.integers(0, N + 1, size=R - 1).tolist())
    offs = [0] + cuts + [N]
    if empty_part and R >= 3:
        offs[2] = offs[1]                   # partition 1 is empty
    mask = (rng.random((B, N)) > 0.3).astype(np.uint8) if masked else None
    if mask is not None:
        mask[:, 0] = 1
    return Q, K, V, offs, mask


def _states(Op, Lp):
    return [ref.state_of(Op[r], Lp[r]) for r in range(len(Lp))]


# ---------------------------------------------------------------- exercise 1
def test_exercise1_ring_and_tree_agree_with_closed_form():
    g = json.load(open(os.path.join(GOLD, "exercise1_ring_tree.json")))
    pairs = g["pairs"]
    m_exp = g["expected"]["m"]
    l_exp = sum(c * math.exp(e) for e, c in g["expected"]["l_exp_terms"])
    # (m, l) states with a one-dimensional dummy accumulator
    states = [(np.array(float(m)), np.array(float(l)), np.zeros(1)) for m, l in pairs]
    for fold in (ref.fold_left, ref.fold_tree):
        m, l, _ = fold(states)
        assert float(m) == m_exp
        assert abs(float(l) - l_exp) <= 1e-15 * l_exp
    bm, bl = brute.merge_ml(pairs)
    assert float(bm) == m_exp and abs(float(bl) - l_exp) <= 1e-15 * l_exp
    # The same states in the (O_r, L_r) form: L_i = m_i + ln l_i, O_i = e_i.
    R = len(pairs)
    L_part = np.array([m + math.log(l) for m, l in pairs])[:, None]          # [R, rows=1]
    O_part = np.eye(R)[:, None, :]                                              # [R, 1, D=R]
    alpha = np.array([l * math.exp(m - m_exp) for m, l in pairs]) / l_exp
    for merge in (ref.merge_oneshot, ref.merge_tree, ref.merge_leftfold):
        Z, L = merge(O_part, L_part)
        np.testing.assert_allclose(Z[0], alpha, rtol=1e-13, atol=0)
        assert abs(L[0] - (m_exp + math.log(l_exp))) < 1e-13


# ------------------------------------------------- semigroup / identity / E4
def _random_tree_fold(states, rnd):
    if len(states) == 1:
        return states[0]
    k = rnd.randint(1, len(states) - 1)
    return ref.merge_states(_random_tree_fold(states[:k], rnd), _random_tree_fold(states[k:], rnd))


def test_merge_any_order_and_grouping():
    rng = np.random.default_rng(7)
    R, rows, D = 13, 6, 5
    O = rng.standard_normal((R, rows, D))
    L = rng.standard_normal((R, rows)) * 4
    L[3] = -np.inf
    O[3] = 0.0
    L[7, 2] = -np.inf
    O[7, 2] = 0.0
    Z0, L0 = ref.merge_oneshot(O, L)
    rnd = random.Random(3)
    for _ in range(20):
        perm = list(range(R))
        rnd.shuffle(perm)
        st = _states(O[perm], L[perm])
        Z1, L1 = ref.finish_state(_random_tree_fold(st, rnd))
        np.testing.assert_allclose(Z1, Z0, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(L1, L0, rtol=1e-12, atol=1e-14)
    for merge in (ref.merge_tree, ref.merge_leftfold):
        Z1, L1 = merge(O, L)
        np.testing.assert_allclose(Z1, Z0, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(L1, L0, rtol=1e-12, atol=1e-14)


def test_empty_state_is_identity():
    rng = np.random.default_rng(8)
    R, rows, D = 5, 4, 3
    O = rng.standard_normal((R, rows, D))
    L = rng.standard_normal((R, rows))
    Z0, L0 = ref.merge_tree(O, L)
    for pos in (0, 2, 5):
        O2 = np.insert(O, pos, 0.0, axis=0)
        L2 = np.insert(L, pos, -np.inf, axis=0)
        for merge in (ref.merge_oneshot, ref.merge_tree, ref.merge_leftfold):
            Z1, L1 = merge(O2, L2)
            np.testing.assert_allclose(Z1, Z0, rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(L1, L0, rtol=1e-13, atol=1e-15)
    # all empty -> (0, -inf), no NaN
    Z, Lz = ref.merge_tree(np.zeros((3, 2, 2)), np.full((3, 2), -np.inf))
    assert np.all(Z == 0) and np.all(np.isneginf(Lz))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_merge_of_partitions_equals_global(seed):
    """eq. 23 reproduces eq. 18: merging the shard states gives the global Z, L."""
    rng = np.random.default_rng(seed)
    Q, K, V, offs, mask = _rand_problem(rng, R=7, qscale=2.0)
    out = ref.encode_ref(Q, K, V, offs, mask, 0.3)
    for merge in (ref.merge_oneshot, ref.merge_tree, ref.merge_leftfold):
        Z, L = merge(out["O_part"], out["L_part"])
        np.testing.assert_allclose(Z, out["Z"], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(L, out["L"], rtol=1e-12, atol=1e-13)


def test_empty_partition_exact_values():
    rng = np.random.default_rng(9)
    Q, K, V, offs, mask = _rand_problem(rng, R=4)
    assert offs[1] == offs[2]
    out = ref.encode_ref(Q, K, V, offs, mask, 0.25)
    assert np.all(np.isneginf(out["L_part"][1]))
    assert np.all(out["O_part"][1] == 0) and not np.any(np.signbit(out["O_part"][1]))
    # a partition whose tokens are all masked behaves the same way
    mask2 = np.ones((2, 40), np.uint8)
    mask2[:, offs[2]:offs[3]] = 0
    out2 = ref.encode_ref(Q, K, V, offs, mask2, 0.25)
    if offs[3] > offs[2]:
        assert np.all(np.isneginf(out2["L_part"][2])) and np.all(out2["O_part"][2] == 0)


# --------------------------------------------------------- closed forms
def test_uniform_scores_give_mean_of_v():
    rng = np.random.default_rng(10)
    Q, K, V, offs, mask = _rand_problem(rng, R=5)
    Q = np.zeros_like(Q)
    out = ref.encode_ref(Q, K, V, offs, mask, 0.125)
    for b in range(2):
        valid = mask[b].astype(bool)
        for h in range(2):
            np.testing.assert_allclose(out["Z"][b, h], np.broadcast_to(V[b, h][valid].mean(0), (5, 8)),
                                       rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(out["L"][b, h], np.log(valid.sum()), rtol=1e-14)
            for r in range(5):
                sel = np.zeros(40, bool)
                sel[offs[r]:offs[r + 1]] = True
                sel &= valid
                if sel.sum() == 0:
                    assert np.all(np.isneginf(out["L_part"][r, b, h]))
                    continue
                np.testing.assert_allclose(out["O_part"][r, b, h],
                                           np.broadcast_to(V[b, h][sel].mean(0), (5, 8)),
                                           rtol=1e-12, atol=1e-14)
                np.testing.assert_allclose(out["L_part"][r, b, h], np.log(sel.sum()), rtol=1e-14)


def test_single_valid_key():
    rng = np.random.default_rng(11)
    Q, K, V, offs, _ = _rand_problem(rng, R=4, masked=False)
    mask = np.zeros((2, 40), np.uint8)
    n_star = 37
    r = max(i for i in range(4) if offs[i] <= n_star < offs[i + 1])
    mask[:, n_star] = 1
    s = 0.3
    out = ref.encode_ref(Q, K, V, offs, mask, s)
    for b in range(2):
        for h in range(2):
            assert np.array_equal(out["O_part"][r, b, h], np.broadcast_to(V[b, h, n_star], (5, 8)))
            np.testing.assert_allclose(out["L_part"][r, b, h], s * (Q[h] @ K[b, h, n_star]), rtol=1e-14)
            assert np.array_equal(out["Z"][b, h], np.broadcast_to(V[b, h, n_star], (5, 8)))


# ------------------------------------------------------- library routines
def _sdpa64(q, k, v, scale, attn_mask=None):
    return F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                          attn_mask=attn_mask, scale=scale).numpy()


def test_single_partition_matches_torch_sdpa_and_logsumexp():
    rng = np.random.default_rng(12)
    Q, K, V, _, mask = _rand_problem(rng, R=2, M=7, N=33, D=16, qscale=3.0)
    s = 0.25
    out = ref.encode_ref(Q, K, V, [0, 33], mask, s)
    qb = np.broadcast_to(Q, (2,) + Q.shape).copy()
    am = torch.from_numpy(mask.astype(bool))[:, None, None, :]
    np.testing.assert_allclose(out["Z"], _sdpa64(qb, K, V, s, am), rtol=1e-11, atol=1e-13)
    S = torch.from_numpy(s * np.einsum("bhmd,bhnd->bhmn", qb, K))
    S = S.masked_fill(~am, float("-inf"))
    np.testing.assert_allclose(out["L"], torch.logsumexp(S, dim=-1).numpy(), rtol=1e-13)
    np.testing.assert_allclose(out["O_part"][0], out["Z"], rtol=0, atol=0)


def test_decode_matches_torch_sdpa():
    rng = np.random.default_rng(13)
    Xq = rng.standard_normal((2, 3, 50, 16))
    Kl = rng.standard_normal((3, 6, 16))
    Z = rng.standard_normal((2, 3, 6, 16))
    Y = ref.decode_ref(Xq, Kl, Z, 0.4)
    Klb = np.broadcast_to(Kl, (2,) + Kl.shape).copy()
    np.testing.assert_allclose(Y, _sdpa64(Xq, Klb, Z, 0.4), rtol=1e-11, atol=1e-13)
    tm = (rng.random((2, 50)) > 0.5).astype(np.uint8)
    Ym = ref.decode_ref(Xq, Kl, Z, 0.4, token_mask=tm)
    assert np.all(Ym[~tm.astype(bool)[:, None, :].repeat(3, 1)] == 0)


def test_flarepp_chain_matches_sdpa_chain():
    rng = np.random.default_rng(14)
    B, H, N, M, D = 1, 2, 64, 4, 8
    Qt = rng.standard_normal((H, M, D))
    Kt, Vt, K, V = (rng.standard_normal((B, H, N, D)) for _ in range(4))
    s = 1 / math.sqrt(D)
    out = ref.flarepp_ref(Qt, Kt, Vt, K, V, [0, 10, 10, 37, 64], s)
    QX = _sdpa64(np.broadcast_to(Qt, (B, H, M, D)).copy(), Kt, Vt, s)
    Z = _sdpa64(QX, K, V, s)
    Y = _sdpa64(K, QX, Z, s)
    np.testing.assert_allclose(out["QX"], QX, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(out["Z"], Z, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(out["Y"], Y, rtol=1e-11, atol=1e-13)


# ------------------------------------------------------------ brute force
def _brute_case(seed):
    rng = np.random.default_rng(100 + seed)
    M, N, D = int(rng.integers(1, 4)), int(rng.integers(1, 13)), int(rng.integers(1, 5))
    R = int(rng.integers(1, 5))
    q = rng.standard_normal((M, D)) * 2
    k = rng.standard_normal((N, D))
    v = rng.standard_normal((N, D))
    offs = [0] + sorted(rng.integers(0, N + 1, size=R - 1).tolist()) + [N]
    valid = (rng.random(N) > 0.3).astype(np.uint8)
    valid[int(rng.integers(0, N))] = 1
    return q, k, v, offs, valid, float(rng.uniform(0.2, 0.9))


@pytest.mark.parametrize("seed", range(6))
def test_encode_and_merge_against_decimal_brute_force(seed):
    q, k, v, offs, valid, s = _brute_case(seed)
    Op, Lp, Z, L = ref.encode_slice(q, k, v, valid, offs, s)
    parts, (bZ, bL) = brute.encode(q.tolist(), k.tolist(), v.tolist(), valid.tolist(), offs, s)
    for r, (bO, bLr) in enumerate(parts):
        for m in range(q.shape[0]):
            if bLr[m] is None:
                assert np.isneginf(Lp[r][m]) and np.all(Op[r][m] == 0)
            else:
                assert abs(Lp[r][m] - float(bLr[m])) <= 1e-13 * max(1, abs(float(bLr[m])))
                np.testing.assert_allclose(Op[r][m], [float(x) for x in bO[m]], rtol=1e-13, atol=1e-14)
    mZ, mL = brute.merge_oneshot(parts)
    for m in range(q.shape[0]):
        np.testing.assert_allclose(Z[m], [float(x) for x in bZ[m]], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(Z[m], [float(x) for x in mZ[m]], rtol=1e-13, atol=1e-14)
        assert abs(L[m] - float(bL[m])) <= 1e-13 * max(1, abs(float(bL[m])))
    # the oracle's own float64 merges of its partition states
    Zt, Lt = ref.merge_tree(np.array(Op), np.array(Lp))
    np.testing.assert_allclose(Zt, np.array([[float(x) for x in row] for row in bZ]), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_decode_against_decimal_brute_force(seed):
    rng = np.random.default_rng(200 + seed)
    n, M, D = 5, int(rng.integers(1, 5)), int(rng.integers(1, 5))
    xq, kl, z = rng.standard_normal((n, D)), rng.standard_normal((M, D)) * 2, rng.standard_normal((M, D))
    y = ref.decode_slice(xq, kl, z, 0.7)
    by = brute.decode(xq.tolist(), kl.tolist(), z.tolist(), 0.7)
    np.testing.assert_allclose(y, np.array([[float(x) for x in r] for r in by]), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("seed", range(4))
def test_backward_against_decimal_brute_force(seed):
    q, k, v, offs, valid, s = _brute_case(seed + 10)
    _, _, Z, L = ref.encode_slice(q, k, v, valid, offs, s)
    dZ = np.random.default_rng(300 + seed).standard_normal(Z.shape)
    dq, dk, dv = ref.encode_bwd_slice(q, k, v, valid, s, Z, L, dZ)
    bq, bk, bv = brute.encode_bwd(q.tolist(), k.tolist(), v.tolist(), valid.tolist(), s, dZ.tolist())
    f = lambda a: np.array([[float(x) for x in r] for r in a])
    np.testing.assert_allclose(dq, f(bq), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk, f(bk), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, f(bv), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- backward
def test_backward_finite_differences():
    rng = np.random.default_rng(15)
    Q, K, V, offs, mask = _rand_problem(rng, B=1, H=1, M=3, N=17, D=4, R=3)
    s = 0.6
    dZ = rng.standard_normal((1, 1, 3, 4))

    def f(Q_, K_, V_):
        return float((ref.encode_ref(Q_, K_, V_, offs, mask, s)["Z"] * dZ).sum())

    out = ref.encode_ref(Q, K, V, offs, mask, s)
    g = ref.encode_bwd_ref(Q, K, V, mask, s, out["Z"], out["L"], dZ)
    h = 1e-6
    for name, X, idxs, G in (("Q", Q, [(0, 0, 0), (0, 2, 3)], g["dQ"][0]),
                             ("K", K, [(0, 0, 1, 2), (0, 0, 16, 0)], g["dK"]),
                             ("V", V, [(0, 0, 4, 1), (0, 0, 9, 3)], g["dV"])):
        for idx in idxs:
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args_p = {"Q": (Xp, K, V), "K": (Q, Xp, V), "V": (Q, K, Xp)}[name]
            args_m = {"Q": (Xm, K, V), "K": (Q, Xm, V), "V": (Q, K, Xm)}[name]
            fd = (f(*args_p) - f(*args_m)) / (2 * h)
            an = G[idx]
            assert abs(fd - an) < 1e-7, (name, idx, fd, an)


def test_backward_matches_torch_autograd_and_local_control_differs():
    rng = np.random.default_rng(16)
    Q, K, V, offs, mask = _rand_problem(rng, B=2, H=2, M=6, N=48, D=8, R=5, qscale=2.0)
    s = 0.35
    dZ = rng.standard_normal((2, 2, 6, 8))
    out = ref.encode_ref(Q, K, V, offs, mask, s)
    g = ref.encode_bwd_ref(Q, K, V, mask, s, out["Z"], out["L"], dZ)
    tq = torch.tensor(np.broadcast_to(Q, (2, 2, 6, 8)).copy(), requires_grad=True)
    tk = torch.tensor(K, requires_grad=True)
    tv = torch.tensor(V, requires_grad=True)
    am = torch.from_numpy(mask.astype(bool))[:, None, None, :]
    Zt = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, scale=s)
    (Zt * torch.from_numpy(dZ)).sum().backward()
    np.testing.assert_allclose(g["dQ"], tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dK"], tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dV"], tv.grad.numpy(), rtol=1e-10, atol=1e-12)
    # masked tokens get exactly zero gradients
    inv = ~mask.astype(bool)
    assert np.all(g["dK"][inv[:, None, :].repeat(2, 1)] == 0)
    assert np.all(g["dV"][inv[:, None, :].repeat(2, 1)] == 0)
    # negative control: a per-partition (locally normalised) backward is different
    dq_l, dk_l, _ = ref.encode_bwd_local_slice(Q[0], K[0, 0], V[0, 0], mask[0], offs, s, dZ[0, 0])
    assert np.abs(dq_l - g["dQ"][0, 0]).max() > 1e-3
    assert np.abs(dk_l - g["dK"][0, 0]).max() > 1e-3


# ------------------------------------------------- permutation / duplication
def test_token_permutation_invariance():
    rng = np.random.default_rng(17)
    Q, K, V, _, mask = _rand_problem(rng, R=2)
    perm = rng.permutation(40)
    a = ref.encode_ref(Q, K, V, [0, 40], mask, 0.3)
    b = ref.encode_ref(Q, K[:, :, perm], V[:, :, perm], [0, 40], mask[:, perm], 0.3)
    np.testing.assert_allclose(a["Z"], b["Z"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(a["L"], b["L"], rtol=1e-13)
    Ya = ref.decode_ref(K, Q, a["Z"], 0.3)
    Yb = ref.decode_ref(K[:, :, perm], Q, b["Z"], 0.3)
    np.testing.assert_allclose(Ya[:, :, perm], Yb, rtol=1e-12, atol=1e-14)


def test_duplicated_tokens_add_ln2():
    """Double counting (the failure mode on the ring-vs-tree page) shifts L by ln 2."""
    rng = np.random.default_rng(18)
    Q, K, V, offs, mask = _rand_problem(rng, R=4)
    a = ref.encode_ref(Q, K, V, offs, mask, 0.3)
    K2, V2 = np.concatenate([K, K], 2), np.concatenate([V, V], 2)
    m2 = np.concatenate([mask, mask], 1)
    b = ref.encode_ref(Q, K2, V2, offs + [o + 40 for o in offs[1:]], m2, 0.3)
    np.testing.assert_allclose(b["Z"], a["Z"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(b["L"] - a["L"], math.log(2), rtol=1e-12)


def test_nan_padding_does_not_leak():
    rng = np.random.default_rng(19)
    Q, K, V, offs, mask = _rand_problem(rng, R=4)
    inv = ~mask.astype(bool)
    K2, V2 = K.copy(), V.copy()
    K2[inv[:, None, :].repeat(2, 1)] = np.nan
    V2[inv[:, None, :].repeat(2, 1)] = np.inf
    a = ref.encode_ref(Q, K, V, offs, mask, 0.3)
    b = ref.encode_ref(Q, K2, V2, offs, mask, 0.3)
    for key in ("O_part", "L_part", "Z", "L"):
        assert np.array_equal(a[key], b[key])
    dZ = rng.standard_normal(a["Z"].shape)
    ga = ref.encode_bwd_ref(Q, K, V, mask, 0.3, a["Z"], a["L"], dZ)
    gb = ref.encode_bwd_ref(Q, K2, V2, mask, 0.3, b["Z"], b["L"], dZ)
    for key in ("dQ", "dK", "dV"):
        assert np.array_equal(ga[key], gb[key])


# ------------------------------------------- decode backward and the FLARE++ chain
def test_decode_backward_matches_torch_autograd():
    """Decode gradients against torch SDPA autograd in float64 (token mask as zero dY rows)."""
    rng = np.random.default_rng(21)
    B, H, N, M, D = 2, 2, 40, 6, 8
    Xq = rng.standard_normal((B, H, N, D))
    Kl = rng.standard_normal((H, M, D)) * 1.5
    Z = rng.standard_normal((B, H, M, D))
    dY = rng.standard_normal((B, H, N, D))
    tm = (rng.random((B, N)) > 0.25).astype(np.uint8)
    s = 0.3
    g = ref.decode_bwd_ref(Xq, Kl, Z, s, dY, token_mask=tm)
    tx = torch.tensor(Xq, requires_grad=True)
    tk = torch.tensor(np.broadcast_to(Kl, (B, H, M, D)).copy(), requires_grad=True)
    tz = torch.tensor(Z, requires_grad=True)
    Y = F.scaled_dot_product_attention(tx, tk, tz, scale=s)
    keep = torch.from_numpy(tm.astype(bool))[:, None, :, None]
    (Y * torch.from_numpy(dY) * keep).sum().backward()
    np.testing.assert_allclose(g["dXq"], tx.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dKlat"], tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dZ"], tz.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.all(g["dXq"][~tm.astype(bool)[:, None, :].repeat(H, 1)] == 0)


def test_decode_backward_finite_differences():
    rng = np.random.default_rng(22)
    xq, kl, z, dy = (rng.standard_normal(sh) for sh in ((9, 4), (3, 4), (3, 4), (9, 4)))
    s = 0.7

    def f(x, k, zz):
        return float((ref.decode_slice(x, k, zz, s) * dy).sum())

    gx, gk, gz = ref.decode_bwd_slice(xq, kl, z, s, dy)
    h = 1e-6
    for which, X, G in (("x", xq, gx), ("k", kl, gk), ("z", z, gz)):
        for idx in ((0, 0), (2, 3), (X.shape[0] - 1, 1)):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args = {"x": lambda A: (A, kl, z), "k": lambda A: (xq, A, z), "z": lambda A: (xq, kl, A)}[which]
            fd = (f(*args(Xp)) - f(*args(Xm))) / (2 * h)
            assert abs(fd - G[idx]) < 1e-7, (which, idx, fd, G[idx])


def test_decode_backward_closed_form_at_uniform_weights():
    """Zero latent keys: every token weighs the M latents equally, so dZ[m] = (1/M) sum_n dY[n]
    and the token queries get no gradient."""
    rng = np.random.default_rng(23)
    xq, dy = rng.standard_normal((11, 5)), rng.standard_normal((11, 5))
    z = rng.standard_normal((4, 5))
    gx, gk, gz = ref.decode_bwd_slice(xq, np.zeros((4, 5)), z, 0.5, dy)
    np.testing.assert_allclose(gz, np.broadcast_to(dy.sum(axis=0) / 4, (4, 5)), rtol=1e-13, atol=1e-14)
    assert np.all(gx == 0)
    # each token's score gradient sums to zero over the latents, so dKlat sums to zero over m
    np.testing.assert_allclose(gk.sum(axis=0), 0.0, atol=1e-12)


def test_flarepp_backward_matches_autograd_through_sdpa_chain():
    """The whole chain's gradients against autograd of Q(X) = SDPA(Qt,Kt,Vt), Z = SDPA(Q(X),K,V),
    Y = SDPA(K, Q(X), Z) in float64 (partitions do not change the exact result)."""
    rng = np.random.default_rng(24)
    B, H, N, M, D = 1, 2, 48, 4, 8
    Qt = rng.standard_normal((H, M, D))
    Kt, Vt, K, V, dY = (rng.standard_normal((B, H, N, D)) for _ in range(5))
    s = 1 / math.sqrt(D)
    g = ref.flarepp_bwd_ref(Qt, Kt, Vt, K, V, [0, 7, 7, 30, 48], s, dY)
    tq = torch.tensor(np.broadcast_to(Qt, (B, H, M, D)).copy(), requires_grad=True)
    tkt, tvt, tk, tv = (torch.tensor(a, requires_grad=True) for a in (Kt, Vt, K, V))
    QX = F.scaled_dot_product_attention(tq, tkt, tvt, scale=s)
    Z = F.scaled_dot_product_attention(QX, tk, tv, scale=s)
    Y = F.scaled_dot_product_attention(tk, QX, Z, scale=s)
    (Y * torch.from_numpy(dY)).sum().backward()
    for name, t in (("dQt", tq), ("dKt", tkt), ("dVt", tvt), ("dK", tk), ("dV", tv)):
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=name)


def test_flarepp_shared_projection_backward_matches_autograd():
    """Shared projections: one K and one V feed the query-synthesis encoder, the
    physical-value encoder and the decoder; autograd sums the three uses itself."""
    rng = np.random.default_rng(25)
    B, H, N, M, D = 1, 2, 40, 4, 8
    Qt = rng.standard_normal((H, M, D))
    K, V, dY = (rng.standard_normal((B, H, N, D)) for _ in range(3))
    s = 1 / math.sqrt(D)
    g = ref.flarepp_shared_bwd_ref(Qt, K, V, [0, 9, 9, 25, 40], s, dY)
    tq = torch.tensor(np.broadcast_to(Qt, (B, H, M, D)).copy(), requires_grad=True)
    tk, tv = (torch.tensor(a, requires_grad=True) for a in (K, V))
    QX = F.scaled_dot_product_attention(tq, tk, tv, scale=s)
    Z = F.scaled_dot_product_attention(QX, tk, tv, scale=s)
    Y = F.scaled_dot_product_attention(tk, QX, Z, scale=s)
    (Y * torch.from_numpy(dY)).sum().backward()
    for name, t in (("dQt", tq), ("dK", tk), ("dV", tv)):
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=name)



def _bf16_straight_through(t):
    """t rounded to bfloat16 in the forward pass, the identity in the backward pass."""
    return t + (t.detach().float().bfloat16().double() - t.detach())


@pytest.mark.parametrize("shared", [False, True])
def test_flarepp_as_executed_chain_matches_autograd_with_bf16_queries(shared):
    """The "as executed" chain (Q(X) consumed as bfloat16 by the physical-value encoder and
    the decoder, its gradient passed through the rounding unchanged) against fp64 autograd
    through the SDPA chain with a straight-through rounding of Q(X).  The query-synthesis
    encoder's backward must use its own unrounded output; a rounded copy in the wrong
    place (encoder 1's saved Z, or one call rounded and the other not) moves the result by
    ~1e-3 relative, far outside the 1e-9 bound."""
    rng = np.random.default_rng(26 + shared)
    B, H, N, M, D = 1, 2, 56, 4, 8
    Qt = rng.standard_normal((H, M, D)) * 2
    Kt, Vt, K, V, dY = (rng.standard_normal((B, H, N, D)) for _ in range(5))
    if shared:
        Kt, Vt = K, V
    s = 1 / math.sqrt(D)
    offs = [0, 11, 11, 40, 56]
    f = ref.flarepp_ref(Qt, Kt, Vt, K, V, offs, s, round_qx_bf16=True)
    g = (ref.flarepp_shared_bwd_ref(Qt, K, V, offs, s, dY, round_qx_bf16=True) if shared else
         ref.flarepp_bwd_ref(Qt, Kt, Vt, K, V, offs, s, dY, round_qx_bf16=True))
    g_plain = (ref.flarepp_shared_bwd_ref(Qt, K, V, offs, s, dY) if shared else
               ref.flarepp_bwd_ref(Qt, Kt, Vt, K, V, offs, s, dY))
    tq = torch.tensor(np.broadcast_to(Qt, (B, H, M, D)).copy(), requires_grad=True)
    tk, tv = (torch.tensor(a, requires_grad=True) for a in (K, V))
    tkt, tvt = (tk, tv) if shared else (torch.tensor(a, requires_grad=True) for a in (Kt, Vt))
    QX = F.scaled_dot_product_attention(tq, tkt, tvt, scale=s)
    QXr = _bf16_straight_through(QX)
    Z = F.scaled_dot_product_attention(QXr, tk, tv, scale=s)
    Y = F.scaled_dot_product_attention(tk, QXr, Z, scale=s)
    (Y * torch.from_numpy(dY)).sum().backward()
    np.testing.assert_allclose(f["QX"], QX.detach().numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(f["Z"], Z.detach().numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(f["Y"], Y.detach().numpy(), rtol=1e-11, atol=1e-13)
    names = (("dQt", tq), ("dK", tk), ("dV", tv)) if shared else \
        (("dQt", tq), ("dKt", tkt), ("dVt", tvt), ("dK", tk), ("dV", tv))
    for name, t in names:
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=name)
        # the rounding is visible: the plain chain differs well beyond the bound above
        assert np.abs(g_plain[name] - g[name]).max() > 1e-6, name
