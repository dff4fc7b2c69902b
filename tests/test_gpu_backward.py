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


def _bwd_spike(B, H, N, M, D, a, spikes, decoy, dtype, seed):
    """Q[m] = a e_0 for every latent row; K = a e_0 at the spike tokens and at a padded decoy
    token, 0 elsewhere; V and dZ entries in {-1, 0, 1} (V with at most 4 nonzeros per row).
    Every non-spike weight is exp(-s a^2) <= e^-110 relative, exactly 0 in float32."""
    g = torch.Generator().manual_seed(seed)
    Q = torch.zeros(H, M, D)
    Q[:, :, 0] = a
    K = torch.zeros(B, H, N, D)
    for n in list(spikes) + [decoy]:
        K[:, :, n, 0] = a
    V = torch.zeros(B, H, N, D)
    V[..., :4] = torch.randint(-1, 2, (B, H, N, 4), generator=g).float()
    V = V[..., torch.randperm(D, generator=g)]
    dZ = torch.randint(-1, 2, (B, H, M, D), generator=g).float()
    mask = torch.ones(B, N, dtype=torch.uint8)
    mask[:, decoy] = 0
    mask[:, decoy + 1:decoy + 40] = 0
    return [t.to(dtype).to(DEV) for t in (Q, K, V, dZ)] + [mask.to(DEV)]


# (M, D, amplitude, power-of-two scale with s a^2 >= 110 and s a a power of two)
_SPIKE_SHAPES = [(64, 64, 32.0, 0.125), (128, 64, 32.0, 0.125), (256, 128, 64.0, 0.0625),
                 (128, 16, 32.0, 0.25), (64, 128, 64.0, 0.0625)]


@pytest.mark.parametrize("M,D,a,s", _SPIKE_SHAPES)
def test_backward_spike_pair_is_bit_exact(M, D, a, s):
    """A tied pair of spike tokens n1, n2 (one in each of two partitions) takes all the weight:
    P = 1/2 on both (bf16-exact), c = (dP1 + dP2)/2, so dS[m, n1] = (dP1 - dP2)/4 = -dS[m, n2].
    Expected, with every value and sum exact in bf16 / float32:
        dK[n1] = -dK[n2] = s a sum_m dS[m, n1] e_0,   dV[n1] = dV[n2] = sum_m dZ[m] / 2,
        dQ = 0,  and dK = dV = 0 at every other token, padded slots and the padded decoy included."""
    B, H, N = 2, 2, 900
    n1, n2, decoy = 63, 577, 700
    offs = [0, 100, 100, 600, 900]
    Q, K, V, dZ, mask = _bwd_spike(B, H, N, M, D, a, (n1, n2), decoy, torch.bfloat16, 5 + M + D)
    O, Lp = fl.encode(Q, K, V, offs, mask, s)
    Z, L, _ = fl.lse_merge(O, Lp)
    dQ, dK, dV = fl.encode_bwd(Q, K, V, offs, mask, s, Z, L, dZ)
    torch.cuda.synchronize()
    Vc, dZc = V.double().cpu(), dZ.double().cpu()
    assert torch.equal(Z.double().cpu(), 0.5 * (Vc[:, :, n1] + Vc[:, :, n2])[:, :, None].expand(B, H, M, D))
    dP1 = (dZc * Vc[:, :, n1][:, :, None]).sum(-1)            # [B, H, M]
    dP2 = (dZc * Vc[:, :, n2][:, :, None]).sum(-1)
    dS1 = 0.25 * (dP1 - dP2)
    wantK = torch.zeros(B, H, N, D, dtype=torch.float64)
    wantK[:, :, n1, 0] = s * a * dS1.sum(-1)
    wantK[:, :, n2, 0] = -s * a * dS1.sum(-1)
    wantV = torch.zeros(B, H, N, D, dtype=torch.float64)
    wantV[:, :, n1] = 0.5 * dZc.sum(2)
    wantV[:, :, n2] = 0.5 * dZc.sum(2)
    assert torch.equal(dK.cpu(), wantK.to(torch.bfloat16))
    assert torch.equal(dV.cpu(), wantV.to(torch.bfloat16))
    assert torch.equal(dQ.cpu(), torch.zeros_like(dQ.cpu()))


@pytest.mark.parametrize("M,D,a,s", _SPIKE_SHAPES)
def test_backward_single_spike_c_cancels_dP(M, D, a, s):
    """One spike token alone: Z = V[n1] exactly, so c = dP[m, n1] and dS = P (dP - c) = 0 exactly
    whatever P's last bit: dK = 0 and dQ = 0 everywhere, dV[n1] = sum_m dZ[m] (P = 1 in bf16)."""
    B, H, N = 1, 3, 700
    n1, decoy = 411, 64
    offs = [0, 300, 700]
    Q, K, V, dZ, mask = _bwd_spike(B, H, N, M, D, a, (n1,), decoy, torch.bfloat16, 7 + M + D)
    O, Lp = fl.encode(Q, K, V, offs, mask, s)
    Z, L, _ = fl.lse_merge(O, Lp)
    dQ, dK, dV = fl.encode_bwd(Q, K, V, offs, mask, s, Z, L, dZ)
    torch.cuda.synchronize()
    assert torch.equal(Z.cpu(), V.float().cpu()[:, :, n1][:, :, None].expand(B, H, M, D))
    assert torch.equal(dK.cpu(), torch.zeros_like(dK.cpu()))
    assert torch.equal(dQ.cpu(), torch.zeros_like(dQ.cpu()))
    wantV = torch.zeros(B, H, N, D, dtype=torch.float64)
    wantV[:, :, n1] = dZ.double().cpu().sum(2)
    assert torch.equal(dV.cpu(), wantV.to(torch.bfloat16))


def test_backward_spike_pair_fp32_vector_path():
    """The float32 vector path with the tied pair: P is float32 (not rounded), so the values carry
    P's rounding, but the index handling is still exact: dV[n1] == dV[n2] and dK[n1] == -dK[n2]
    bit for bit, dQ == 0 and every other token's gradient == 0 exactly.  The values: P = exp(S - L)
    with L = s a^2 + ln 2 = 181.7, whose float32 spacing is 1.5e-5, so P (and every gradient value)
    carries a relative error of that order; they are checked to 3e-5 relative."""
    B, H, N, M, D, a, s = 1, 2, 1024, 16, 32, 32.0, float(np.float32(32 ** -0.5))
    n1, n2, decoy = 299, 300, 900          # both sides of the 300 | 200 partition edge
    offs = [0, 300, 500, 924, 1024]
    Q, K, V, dZ, mask = _bwd_spike(B, H, N, M, D, a, (n1, n2), decoy, torch.float32, 11)
    O, Lp = fl.encode(Q, K, V, offs, mask, s)
    Z, L, _ = fl.lse_merge(O, Lp)
    dQ, dK, dV = fl.encode_bwd(Q, K, V, offs, mask, s, Z, L, dZ)
    torch.cuda.synchronize()
    others = torch.ones(N, dtype=torch.bool)
    others[[n1, n2]] = False
    dKc, dVc = dK.cpu(), dV.cpu()
    assert (dKc[:, :, others] == 0).all() and (dVc[:, :, others] == 0).all()
    assert torch.equal(dVc[:, :, n1], dVc[:, :, n2])
    assert torch.equal(dKc[:, :, n1], -dKc[:, :, n2])
    assert (dKc[..., 1:] == 0).all()
    assert torch.equal(dQ.cpu(), torch.zeros_like(dQ.cpu()))
    e = ref.encode_ref(Q, K, V, offs, mask, s)
    gr = ref.encode_bwd_ref(Q, K, V, mask, s, e["Z"], e["L"], dZ)
    compare(dK, gr["dK"], "dK", 1e-5, rtol=3e-5)
    compare(dV, gr["dV"], "dV", 1e-5, rtol=3e-5)


def test_backward_is_deterministic():
    w, x = _masked_case(128, 64, N=2048, R=4, wid=970)
    a = _run(w, x)
    b = _run(w, x)
    for u, v in zip(a[2:], b[2:]):
        assert torch.equal(u, v)


@pytest.mark.parametrize("M,D", [(128, 64), (256, 128), (128, 16)])
def test_launch_order_changes_no_bit(M, D):
    """Masked inputs launch their chunks heaviest first (by valid-token count), so
    permuting the batch rows permutes the launch order.  Each chunk writes its own
    state and query-gradient partial, which the reduce sums in chunk order, so the
    forward states and all gradients come out as the same bits, permuted."""
    w, x = _masked_case(M, D, N=16384, R=4, B=3, wid=1990)
    perm = [2, 0, 1]
    y = dict(x)
    for k in ("K", "V", "dZ"):
        y[k] = x[k][perm].contiguous()
    y["mask"] = x["mask"][perm].contiguous()
    outs = []
    for inp in (x, y):
        O, Lp = fl.encode(inp["Q"], inp["K"], inp["V"], w.offsets, inp["mask"], w.scale)
        outs.append((O, Lp) + _run(w, inp))
    torch.cuda.synchronize()
    (O0, L0, Z0, Lg0, dQ0, dK0, dV0), (O1, L1, Z1, Lg1, dQ1, dK1, dV1) = outs
    assert torch.equal(O0[:, perm], O1) and torch.equal(L0[:, perm], L1)
    assert torch.equal(Z0[perm], Z1) and torch.equal(Lg0[perm], Lg1)
    assert torch.equal(dQ0[perm], dQ1) and torch.equal(dK0[perm], dK1) and torch.equal(dV0[perm], dV1)
    _check(w, x, *outs[0][2:])
