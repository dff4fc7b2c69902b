"""GPU parity of lse_merge on crafted partition states (not encoder output).

"Ring vs. Tree Attention": the online-softmax merge of (m, l) states, the
balanced-tree schedule and the core exercise of its Exercises section;
"FLARE++" appendix: the (O_r, L_r) form of a shard's state, the empty state
(0, -inf) and the max-stabilised merge.  The states here have log-normalisers
spread over +-80, empty leaves anywhere (rows empty in every leaf included) and
R from 1 to 300, which the encoder's own output never exercises.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import split_kv_softmax_amd as fl
from oracle import flare_ref as ref
from tests._util import compare, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_exercise1_through_the_api():
    """The eight (m_i, l_i) pairs of the core exercise as (O_i, L_i) = (e_i, m_i + ln l_i), D = 8:
    the merged Z is the vector of shard masses alpha_i = l_i e^(m_i - m) / l and L = m + ln l,
    with m = 4 and l = 1 + e^-1 + 5e^-2 + 10e^-3 + 8e^-4 (worked out by hand in the fixture)."""
    g = json.load(open(os.path.join(GOLD, "exercise1_ring_tree.json")))
    pairs = g["pairs"]
    m_exp = g["expected"]["m"]
    l_exp = sum(c * math.exp(e) for e, c in g["expected"]["l_exp_terms"])
    R = len(pairs)
    L_part = torch.tensor([[m + math.log(l)] for m, l in pairs], dtype=torch.float32, device=DEV)   # [R, 1]
    O_part = torch.eye(R, dtype=torch.float32, device=DEV)[:, None, :].contiguous()                  # [R, 1, 8]
    Z, L, Zb = fl.lse_merge(O_part, L_part, want_bf16=True)
    torch.cuda.synchronize()
    alpha = np.array([l * math.exp(m - m_exp) for m, l in pairs]) / l_exp
    np.testing.assert_allclose(to64(Z[0]), alpha, rtol=0, atol=1e-6)
    assert abs(float(L[0]) - (m_exp + math.log(l_exp))) <= 1e-6
    assert torch.equal(Zb, Z.to(torch.bfloat16))


def _crafted(R, rows, D, seed, spread=80.0, p_empty=0.25):
    g = np.random.default_rng(seed)
    L = g.uniform(-spread, spread, size=(R, rows)).astype(np.float32)
    empty = g.random((R, rows)) < p_empty
    empty[:, 0] = True                         # row 0: empty in every leaf
    if rows > 1:
        empty[:, 1] = True
        empty[R // 2, 1] = False               # row 1: one live leaf, in the middle
    if rows > 2:
        empty[0, 2] = True                     # row 2: the first leaf empty
    L[empty] = -np.inf
    O = g.standard_normal((R, rows, D)).astype(np.float32)
    O[empty] = 0.0
    return torch.from_numpy(O).to(DEV), torch.from_numpy(L).to(DEV)


@pytest.mark.parametrize("R", [1, 2, 3, 16, 17, 64, 300])
def test_crafted_states_against_oracle_tree(R):
    """Wide L spreads, empty leaves and globally empty rows against the oracle's balanced tree
    (and its one-shot and left-fold forms) on the same float32 states widened to float64."""
    rows, D = 45, 64
    O, Lp = _crafted(R, rows, D, 40 + R)
    Z, L, Zb = fl.lse_merge(O, Lp, want_bf16=True)
    torch.cuda.synchronize()
    O64, L64 = to64(O), to64(Lp)
    for merge in (ref.merge_tree, ref.merge_oneshot, ref.merge_leftfold):
        Zr, Lr = merge(O64, L64)
        compare(Z, Zr, f"Z {merge.__name__}", 1e-5)
        compare(L, Lr, f"L {merge.__name__}", 1e-5, rtol=2e-7)
    Zc, Lc = Z.cpu(), L.cpu()
    assert torch.isneginf(Lc[0]) and (Zc[0] == 0).all() and not torch.signbit(Zc[0]).any()
    if rows > 1:
        # one live leaf: the merge returns its state (L exactly; O up to the 1/l with l = 1)
        assert float(Lc[1]) == float(Lp[R // 2, 1])
        assert torch.equal(Zc[1], O[R // 2, 1].cpu())
    assert not torch.isnan(Zc).any() and not torch.isnan(Lc).any()
    assert torch.equal(Zb, Z.to(torch.bfloat16))


@pytest.mark.parametrize("R", [5, 64])
def test_crafted_states_any_order(R):
    """The semigroup proposition on the GPU: permuting the leaves changes the result only by
    rounding (float32, max-abs 1e-5 on Z, 1e-5 + 2e-7 |L| on L)."""
    rows, D = 33, 32
    O, Lp = _crafted(R, rows, D, 90 + R)
    perm = torch.from_numpy(np.random.default_rng(R).permutation(R)).to(DEV)
    Z1, L1, _ = fl.lse_merge(O, Lp)
    Z2, L2, _ = fl.lse_merge(O[perm].contiguous(), Lp[perm].contiguous())
    torch.cuda.synchronize()
    compare(Z2, to64(Z1), "Z permuted", 1e-5)
    compare(L2, to64(L1), "L permuted", 1e-5, rtol=2e-7)
