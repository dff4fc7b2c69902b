"""GPU parity of the encoder backward (global statistics) against the CPU oracle.

The backward takes the forward's global Z and L.  Two comparisons per case:
end to end (the oracle's own Z, L) and isolated (the GPU's Z, L widened and
fed to the oracle's backward, so forward rounding does not mix in).
"""
import numpy as np
import pytest
import torch

import split_kv_softmax_amd as fl
import workloads as W
from oracle import flare_ref as ref
from tests._util import compare, compare_bf16, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _masked_case(M, D, N, R, B=2, H=2, dtype="bf16", wid=900):
    slot = N // R
    w = W.MASKED_FWD_BWD.with_(name=f"bwd_M{M}_D{D}_N{N}", wid=wid + M + D, dtype=dtype, B=B, H=H, N=slot * R, M=M,
                               D=D, offsets=W.equal_offsets(slot * R, R), mask_slot=slot,
                               q_std=float(D ** -0.5))
    return w, w.make(DEV)


def _run(w, x):
    O, Lp = fl.encode(x["Q"], x["K"], x["V"], w.offsets, x.get("mask"), w.scale)
    Z, L, _ = fl.lse_merge(O, Lp)
    dQ, dK, dV = fl.encode_bwd(x["Q"], x["K"], x["V"], w.offsets, x.get("mask"), w.scale, Z, L, x["dZ"])
    torch.cuda.synchronize()
    return Z, L, dQ, dK, dV


def _check(w, x, Z, L, dQ, dK, dV, fp32=False):
    e = ref.encode_ref(x["Q"], x["K"], x["V"], w.offsets, x.get("mask"), w.scale)
    g_end = ref.encode_bwd_ref(x["Q"], x["K"], x["V"], x.get("mask"), w.scale, e["Z"], e["L"], x["dZ"])
    g_iso = ref.encode_bwd_ref(x["Q"], x["K"], x["V"], x.get("mask"), w.scale, Z, L, x["dZ"])
    for g, tag in ((g_iso, "isolated"), (g_end, "end-to-end")):
        if fp32:
            for k, t in (("dQ", dQ), ("dK", dK), ("dV", dV)):
                compare(t, g[k], f"{k} {tag}", 1e-5)
        else:
            compare_bf16(dQ, g["dQ"], f"dQ {tag}")
            compare_bf16(dK, g["dK"], f"dK {tag}")
            compare_bf16(dV, g["dV"], f"dV {tag}")
    if "mask" in x:
        inv = (x["mask"] == 0)[:, None, :, None].expand_as(dK)
        assert (dK[inv] == 0).all() and (dV[inv] == 0).all()


# every matrix-core shape: fused (one pass) and split (separate query-gradient pass)
@pytest.mark.parametrize("M,D", [(32, 64), (64, 64), (128, 64), (256, 64),
                                 (32, 128), (64, 128), (128, 128), (256, 128), (32, 16), (64, 16), (128, 16)])
def test_backward_masked_bf16(M, D):
    w, x = _masked_case(M, D, N=2048, R=4)
    _check(w, x, *_run(w, x))


def test_backward_padding_contents_do_not_matter():
    """NaN in masked K/V rows changes nothing: the gradients are bitwise those of clean padding."""
    w, x = _masked_case(128, 64, N=2048, R=4, wid=980)
    a = _run(w, x)
    inv = (x["mask"] == 0)[:, None, :, None].expand_as(x["K"])
    y = dict(x)
    y["K"] = x["K"].masked_fill(inv, float("nan"))
    y["V"] = x["V"].masked_fill(inv, float("nan"))
    O, Lp = fl.encode(y["Q"], y["K"], y["V"], w.offsets, y["mask"], w.scale)
    Z, L, _ = fl.lse_merge(O, Lp)
    assert torch.equal(Z, a[0]) and torch.equal(L, a[1])
    g = fl.encode_bwd(y["Q"], y["K"], y["V"], w.offsets, y["mask"], w.scale, a[0], a[1], y["dZ"])
    torch.cuda.synchronize()
    for u, v in zip(g, a[2:]):
        assert torch.equal(u, v)


def test_backward_many_chunks_ragged_tail():
    """One (b, h) slice, so the tokens split into many chunks; N is not a multiple of 64."""
    w, x = _masked_case(128, 64, N=40000, R=7, B=1, H=1, wid=990)
    _check(w, x, *_run(w, x))


def test_backward_fp32():
    w, x = _masked_case(24, 32, N=900, R=3, dtype="f32")
    _check(w, x, *_run(w, x), fp32=True)


def test_backward_unmasked_ragged_bf16():
    base = W.shrink(W.FLAREPP, 3000, R=5, H=2, ragged=True)
    Q = W.normal((2, 128, 64), 950, W.T_Q, 1 / 8, torch.bfloat16, DEV)
    K = W.normal((1, 2, 3000, 64), 950, W.T_K, 1.0, torch.bfloat16, DEV)
    V = W.normal((1, 2, 3000, 64), 950, W.T_V, 1.0, torch.bfloat16, DEV)
    dZ = W.normal((1, 2, 128, 64), 950, W.T_DZ, 1.0, torch.bfloat16, DEV)
    x = {"Q": Q, "K": K, "V": V, "dZ": dZ}
    _check(base, x, *_run(base, x))


@pytest.mark.parametrize("M", [64, 128])
def test_backward_head_dim_16_unmasked_ragged(M):
    """Head dim 16 without a mask, ragged partitions and a tail that is not a whole tile."""
    base = W.shrink(W.FLAREPP_D16, 3333, R=5, H=2, ragged=True)
    Q = W.normal((2, M, 16), 955 + M, W.T_Q, 0.25, torch.bfloat16, DEV)
    K = W.normal((1, 2, 3333, 16), 955 + M, W.T_K, 1.0, torch.bfloat16, DEV)
    V = W.normal((1, 2, 3333, 16), 955 + M, W.T_V, 1.0, torch.bfloat16, DEV)
    dZ = W.normal((1, 2, M, 16), 955 + M, W.T_DZ, 1.0, torch.bfloat16, DEV)
    x = {"Q": Q, "K": K, "V": V, "dZ": dZ}
    _check(base, x, *_run(base, x))


def test_backward_stress_scores_bf16():
    w, x = _masked_case(128, 64, N=2048, R=4, wid=960)
    x["Q"] = (x["Q"].float() * 32).to(torch.bfloat16)     # score spread ~4
    _check(w, x, *_run(w, x))


def test_backward_only_attended_tokens_get_gradients():
    """One latent direction hits two tied spike tokens; every other weight underflows to 0,
    so every other token's dK and dV must be exactly zero, and dV of the pair equals half
    the column sum of dZ."""
    B, H, N, M, D = 1, 2, 640, 64, 64
    a = 32.0
    Q = torch.zeros(H, M, D)
    Q[:, :, 0] = a
    K = torch.zeros(B, H, N, D)
    n1, n2 = 63, 577
    K[:, :, n1, 0] = a
    K[:, :, n2, 0] = a
    g = torch.Generator().manual_seed(5)
    V = torch.randint(-1, 2, (B, H, N, D), generator=g).float()
    dZ = torch.randint(-1, 2, (B, H, M, D), generator=g).float()
    Q, K, V, dZ = (t.to(torch.bfloat16).to(DEV) for t in (Q, K, V, dZ))
    offs = [0, 100, 100, 600, 640]
    O, Lp = fl.encode(Q, K, V, offs)
    Z, L, _ = fl.lse_merge(O, Lp)
    dQ, dK, dV = fl.encode_bwd(Q, K, V, offs, None, None, Z, L, dZ)
    torch.cuda.synchronize()
    others = torch.ones(N, dtype=torch.bool)
    others[[n1, n2]] = False
    assert (dK[:, :, others] == 0).all() and (dV[:, :, others] == 0).all()
    half_sum = 0.5 * dZ.float().sum(dim=2)                           # [B,H,D]
    torch.testing.assert_close(dV[:, :, n1].float(), half_sum, rtol=1e-2, atol=1e-2)
    torch.testing.assert_close(dV[:, :, n2].float(), half_sum, rtol=1e-2, atol=1e-2)
    torch.testing.assert_close(dK[:, :, n1].float(), -dK[:, :, n2].float(), rtol=1e-2, atol=1e-3)
    # only the first head dim of dK can be nonzero (the scores only see direction 0)
    assert (dK[:, :, :, 1:] == 0).all()


def test_backward_is_deterministic():
    w, x = _masked_case(128, 64, N=2048, R=4, wid=970)
    a = _run(w, x)
    b = _run(w, x)
    for u, v in zip(a[2:], b[2:]):
        assert torch.equal(u, v)


@pytest.mark.parametrize("M,D", [(128, 64), (256, 128), (128, 16)])
def test_heavy_first_launch_order_changes_no_bit(M, D, monkeypatch):
    """Masked inputs launch their chunks heaviest first; each chunk writes its own
    state and partial, so the forward states and all gradients are the same bits
    with the plain block order."""
    w, x = _masked_case(M, D, N=16384, R=4, B=3, wid=1990)
    outs = []
    for flag in ("1", "0"):
        monkeypatch.setenv("FLARE_HEAVY_FIRST", flag)
        O, Lp = fl.encode(x["Q"], x["K"], x["V"], w.offsets, x["mask"], w.scale)
        outs.append((O, Lp) + _run(w, x))
    torch.cuda.synchronize()
    for u, v in zip(*outs):
        assert torch.equal(u, v)
    _check(w, x, *outs[0][2:])
