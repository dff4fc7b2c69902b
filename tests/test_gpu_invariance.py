"""GPU invariance tests: properties of the exact split softmax that hold at any
size, checked on the HIP path alone (one arrangement against another).

* Any grouping of the tokens into disjoint partitions, with empty partitions
  inserted or a single partition, gives the same merged (Z, L): the merge is
  associative and commutative ("Ring vs. Tree Attention", the semigroup
  proposition; FLARE++ appendix on context parallelism, the exact merge).
* Permuting the tokens (with their mask bits) changes nothing.
* Every token present twice leaves Z unchanged and raises L by ln 2.
* The decode is unchanged by a permutation of the latent rows applied to
  both the latent keys and Z.
* The encoder backward with the global statistics gives the same gradients
  under any grouping (the between-partition term c makes it exact).

Tolerances: the bf16 parity bounds for outputs; for L a bound from the bf16
rounding of the weights (relative 2^-9 per weight, so at most about 2e-3 on the
log of their sum), 1e-5 for float32 inputs.
"""
import math

import numpy as np
import pytest
import torch

import split_kv_softmax_amd as fl
from tests._util import F32_ATOL, compare, compare_bf16, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"
L_TOL_BF16 = 2.5e-3

CASES = [
    # (M, D, masked, dtype): pipelined encoder, general matrix-core encoder with
    # a mask, head dim 16 with a mask, single query, float32 vector path
    (128, 64, False, torch.bfloat16),
    (256, 128, True, torch.bfloat16),
    (64, 16, True, torch.bfloat16),
    (1, 128, False, torch.bfloat16),
    (16, 32, True, torch.float32),
]


def _ids(c):
    return f"M{c[0]}_D{c[1]}_{'masked' if c[2] else 'dense'}_{'bf16' if c[3] == torch.bfloat16 else 'f32'}"


def _inputs(M, D, N, masked, dtype, seed, B=2, H=2):
    g = torch.Generator().manual_seed(seed)
    Q = (torch.randn((H, M, D), generator=g) * D ** -0.5).to(dtype)
    K = torch.randn((B, H, N, D), generator=g).to(dtype)
    V = torch.randn((B, H, N, D), generator=g).to(dtype)
    mask = None
    if masked:
        mask = (torch.rand((B, N), generator=g) > 0.4).to(torch.uint8)
        mask[:, 0] = 1
    return Q, K, V, mask


def _merged(Q, K, V, offsets, mask, scale):
    dev = lambda t: None if t is None else t.to(DEV)
    O, Lp = fl.encode(dev(Q), dev(K), dev(V), offsets, dev(mask), scale)
    Z, L, _ = fl.lse_merge(O, Lp)
    torch.cuda.synchronize()
    return Z, L


def _same(a, b, f32, what):
    (Za, La), (Zb, Lb) = a, b
    if f32:
        compare(Zb, to64(Za), f"Z {what}", F32_ATOL)
    else:
        compare_bf16(Zb, to64(Za), f"Z {what}")
    compare(Lb, to64(La), f"L {what}", F32_ATOL if f32 else L_TOL_BF16)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_any_grouping_of_the_tokens_gives_the_same_merge(case):
    M, D, masked, dtype = case
    N = 4100
    print(f"case {_ids(case)} N={N}", flush=True)
    Q, K, V, mask = _inputs(M, D, N, masked, dtype, seed=31 + M + D)
    s = fl.scale_for(D)
    f32 = dtype == torch.float32
    base = _merged(Q, K, V, [0, 1500, 2900, N], mask, s)
    for offs in ([0, N],                                   # one partition
                 [0, 0, 64, 64, 700, 2049, 2049, 3333, N],  # empty partitions inserted, tile-crossing cuts
                 [0] + list(range(97, N, 613)) + [N]):     # many short ragged ones
        _same(base, _merged(Q, K, V, offs, mask, s), f32, f"R={len(offs) - 1}")


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_token_permutation_changes_nothing(case):
    M, D, masked, dtype = case
    N = 3000
    print(f"case {_ids(case)} N={N}", flush=True)
    Q, K, V, mask = _inputs(M, D, N, masked, dtype, seed=57 + M + D)
    s = fl.scale_for(D)
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(9))
    Kp, Vp = K[:, :, perm].contiguous(), V[:, :, perm].contiguous()
    mp = None if mask is None else mask[:, perm].contiguous()
    offs = [0, 1000, 1000, 2222, N]
    _same(_merged(Q, K, V, offs, mask, s), _merged(Q, Kp, Vp, offs, mp, s), dtype == torch.float32, "permuted")


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_every_token_twice_adds_ln2(case):
    M, D, masked, dtype = case
    N = 2500
    print(f"case {_ids(case)} N={N}", flush=True)
    Q, K, V, mask = _inputs(M, D, N, masked, dtype, seed=83 + M + D)
    s = fl.scale_for(D)
    f32 = dtype == torch.float32
    Z, L = _merged(Q, K, V, [0, 900, N], mask, s)
    K2, V2 = torch.cat([K, K], dim=2), torch.cat([V, V], dim=2)
    m2 = None if mask is None else torch.cat([mask, mask], dim=1)
    Z2, L2 = _merged(Q, K2, V2, [0, 900, 2 * N - 300, 2 * N], m2, s)
    if f32:
        compare(Z2, to64(Z), "Z doubled", F32_ATOL)
    else:
        compare_bf16(Z2, to64(Z), "Z doubled")
    compare(L2, to64(L) + math.log(2.0), "L doubled", F32_ATOL if f32 else L_TOL_BF16)


@pytest.mark.parametrize("M,D", [(128, 64), (64, 128), (64, 16)])
def test_decode_latent_row_permutation(M, D):
    B, H, N = 2, 2, 1500
    g = torch.Generator().manual_seed(101 + M)
    Xq = torch.randn((B, H, N, D), generator=g).to(torch.bfloat16).to(DEV)
    Kl = (torch.randn((H, M, D), generator=g) * 0.5).to(torch.bfloat16).to(DEV)
    Z = (torch.randn((B, H, M, D), generator=g) * 0.1).to(DEV)
    perm = torch.randperm(M, generator=g).to(DEV)
    s = fl.scale_for(D)
    Y = fl.decode(Xq, Kl, Z, s)
    Yp = fl.decode(Xq, Kl[:, perm].contiguous(), Z[:, :, perm].contiguous(), s)
    torch.cuda.synchronize()
    compare_bf16(Yp, to64(Y), "Y with permuted latents")


@pytest.mark.parametrize("M,D,masked", [(128, 64, False), (256, 128, True), (64, 16, True)])
def test_backward_any_grouping_gives_the_same_gradients(M, D, masked):
    N = 3100
    print(f"case M={M} D={D} masked={masked} N={N}", flush=True)
    Q, K, V, mask = _inputs(M, D, N, masked, torch.bfloat16, seed=211 + M + D)
    Q, K, V = Q.to(DEV), K.to(DEV), V.to(DEV)
    mask = None if mask is None else mask.to(DEV)
    s = fl.scale_for(D)
    dZ = (torch.randn((2, 2, M, D), generator=torch.Generator().manual_seed(5))).to(torch.bfloat16).to(DEV)
    grads = []
    for offs in ([0, 1200, N], [0, N], [0, 0, 333, 333, 1900, 2047, N]):
        O, Lp = fl.encode(Q, K, V, offs, mask, s)
        Z, L, _ = fl.lse_merge(O, Lp)
        dQ = torch.empty((2, 2, M, D), dtype=torch.float32, device=DEV)
        dK, dV = torch.empty_like(K), torch.empty_like(V)
        fl.encode_bwd(Q, K, V, offs, mask, s, Z, L, dZ, dQ, dK, dV)
        torch.cuda.synchronize()
        grads.append((dQ, dK, dV))
    for i in (1, 2):
        for name, a, b in zip(("dQ", "dK", "dV"), grads[0], grads[i]):
            compare_bf16(b, to64(a), f"{name} grouping {i}")
