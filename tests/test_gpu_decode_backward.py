"""GPU parity of the decode backward and the FLARE++ backward chain against the CPU oracle.

The decode backward takes the forward's latents (Klat, Z) and the token
queries; the chain runs the decoder backward, the physical-value encoder
backward (adding into the decoder's query and key gradients) and the
query-synthesis encoder backward, each with its own saved statistics.
"""
import numpy as np
import pytest
import torch

import split_kv_softmax_amd as fl
import workloads as W
from oracle import flare_ref as ref
from tests._util import compare, compare_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _decode_case(M, D, N, B=2, H=2, dtype=torch.bfloat16, wid=1200, masked=True, per_batch=False):
    w = wid + M + D
    Xq = W.normal((B, H, N, D), w, W.T_K, 1.0, dtype, DEV)
    Kl = W.normal((B, H, M, D) if per_batch else (H, M, D), w, W.T_Q, D ** -0.5 * 2, dtype, DEV)
    Z = W.normal((B, H, M, D), w, W.T_V, 1.0, torch.float32, DEV)
    dY = W.normal((B, H, N, D), w, W.T_DZ, 1.0, dtype, DEV)
    tm = None
    if masked:
        g = np.random.default_rng(w)
        m = (g.random((B, N)) > 0.2).astype(np.uint8)
        m[:, 0] = 1
        tm = torch.from_numpy(m).to(DEV)
    return Xq, Kl, Z, dY, tm


def _check_decode(Xq, Kl, Z, dY, tm, scale, fp32=False, with_cast=False):
    B, H, N, D = Xq.shape
    M = Kl.shape[-2]
    dZc = torch.empty((B, H, M, D), dtype=Xq.dtype, device=DEV) if with_cast else None
    dX, dK, dZ = fl.decode_bwd(Xq, Kl, Z, scale, dY, token_mask=tm, dZ_cast=dZc)
    torch.cuda.synchronize()
    g = ref.decode_bwd_ref(Xq, Kl, Z, scale, dY, token_mask=tm)
    if fp32:
        compare(dX, g["dXq"], "dXq", 1e-5)
        compare(dK, g["dKlat"], "dKlat", 1e-5)
        compare(dZ, g["dZ"], "dZ", 1e-5)
    else:
        compare_bf16(dX, g["dXq"], "dXq")
        compare_bf16(dK, g["dKlat"], "dKlat")
        compare_bf16(dZ, g["dZ"], "dZ")
    if tm is not None:
        inv = (tm == 0)[:, None, :, None].expand_as(dX)
        assert (dX[inv] == 0).all()
    if with_cast:
        assert torch.equal(dZc, dZ.to(Xq.dtype))
    return dX, dK, dZ


def test_decode_backward_fp32():
    Xq, Kl, Z, dY, tm = _decode_case(16, 32, 300, dtype=torch.float32)
    _check_decode(Xq, Kl, Z, dY, tm, 32 ** -0.5, fp32=True)


@pytest.mark.parametrize("M,D", [(32, 64), (64, 64), (128, 64), (32, 128), (64, 128), (128, 128), (256, 64),
                                 (32, 16), (64, 16), (128, 16)])
def test_decode_backward_bf16(M, D):
    Xq, Kl, Z, dY, tm = _decode_case(M, D, 2100)
    _check_decode(Xq, Kl, Z, dY, tm, float(np.float32(1) / np.sqrt(np.float32(D))), with_cast=True)


def test_decode_backward_unmasked_per_batch_latents_ragged_tail():
    Xq, Kl, Z, dY, _ = _decode_case(128, 64, 4999, B=1, H=3, masked=False, per_batch=True)
    _check_decode(Xq, Kl, Z, dY, None, 0.125)


def test_decode_backward_head_dim_16_unmasked_ragged_tail():
    Xq, Kl, Z, dY, _ = _decode_case(128, 16, 4999, B=1, H=3, masked=False, per_batch=True)
    _check_decode(Xq, Kl, Z, dY, None, 0.25)


def test_decode_backward_is_deterministic():
    Xq, Kl, Z, dY, tm = _decode_case(128, 64, 3000, wid=1300)
    a = fl.decode_bwd(Xq, Kl, Z, 0.125, dY, token_mask=tm)
    b = fl.decode_bwd(Xq, Kl, Z, 0.125, dY, token_mask=tm)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_encoder_backward_accumulate_flags_and_cast():
    """ACCUMULATE_DQ / ACCUMULATE_DK add into what is there; dQ_cast is dQ in the input dtype."""
    base = W.shrink(W.FLAREPP, 3000, R=3, H=2, ragged=True)
    x = base.make(DEV)
    Q = W.normal((1, 2, 128, 64), 1400, W.T_Q, 1 / 8, torch.bfloat16, DEV)
    dZ = W.normal((1, 2, 128, 64), 1400, W.T_DZ, 1.0, torch.bfloat16, DEV)
    O, Lp = fl.encode(Q, x["K"], x["V"], base.offsets, None, base.scale)
    Z, L, _ = fl.lse_merge(O, Lp)
    dQ0, dK0, dV0 = fl.encode_bwd(Q, x["K"], x["V"], base.offsets, None, base.scale, Z, L, dZ)
    prevQ = torch.randn_like(dQ0)
    prevK = torch.randn_like(dK0.float()).to(torch.bfloat16)
    dQ, dK = prevQ.clone(), prevK.clone()
    dQc = torch.empty_like(dQ0, dtype=torch.bfloat16)
    _, _, dV = fl.encode_bwd(Q, x["K"], x["V"], base.offsets, None, base.scale, Z, L, dZ, dQ=dQ, dK=dK, dQ_cast=dQc,
                             flags=fl.ACCUMULATE_DQ | fl.ACCUMULATE_DK)
    torch.cuda.synchronize()
    assert torch.equal(dQ, prevQ + dQ0)
    assert torch.equal(dK, (prevK.float() + dK0.float()).to(torch.bfloat16))
    assert torch.equal(dV, dV0)
    assert torch.equal(dQc, dQ.to(torch.bfloat16))


def test_flarepp_backward_chain_small():
    """The three-call chain against the oracle's chain with Q(X) rounded to bf16 as the kernels use it."""
    w = W.shrink(W.FLAREPP, 4000, R=4, H=2, ragged=True)
    x = w.make(DEV)
    dY = W.normal((1, 2, 4000, 64), 1500, W.T_DZ, 1.0, torch.bfloat16, DEV)
    fwd = fl.flarepp_forward(x["Qt"], x["Kt"], x["Vt"], x["K"], x["V"], w.offsets, w.scale)
    g = fl.flarepp_backward(fwd, x["Qt"], x["Kt"], x["Vt"], x["K"], x["V"], w.offsets, dY, w.scale)
    torch.cuda.synchronize()
    r = ref.flarepp_bwd_ref(x["Qt"], x["Kt"], x["Vt"], x["K"], x["V"], w.offsets, w.scale, dY, round_qx_bf16=True)
    compare_bf16(g["dQX"], r["dQX"], "dQX")
    for k in ("dQt", "dKt", "dVt", "dK", "dV"):
        compare_bf16(g[k], r[k], k)
    # the plain chain (Q(X) kept in float64) at the same bf16 bounds
    p = ref.flarepp_bwd_ref(x["Qt"], x["Kt"], x["Vt"], x["K"], x["V"], w.offsets, w.scale, dY)
    for k in ("dQX", "dQt", "dKt", "dVt", "dK", "dV"):
        compare_bf16(g[k], p[k], k + " plain")


_BWD_SHAPES = [(32, 64, True), (64, 64, True), (128, 64, False), (256, 64, True), (32, 128, False),
               (64, 128, True), (128, 128, True), (256, 128, True), (32, 16, False), (64, 16, True),
               (128, 16, True), (16, 32, False), (16, 64, True)]


@pytest.mark.parametrize("M,D,masked", _BWD_SHAPES)
def test_encoder_backward_accumulate_flags_every_shape(M, D, masked):
    """ACCUMULATE_DK, ACCUMULATE_DV and both add the gradient to what dK and dV hold
    (bf16 sums of the same bf16 gradient, so bit for bit), on every matrix-core shape of
    the key/value kernel and on the vector path; rows of masked tokens keep their old
    values, and the gradient not accumulated is written as without flags."""
    B, H, N = 2, 2, 2600
    offsets = [0, 900, 900, 2000, 2600]
    dt = torch.bfloat16 if D != 32 else torch.float32
    Q = W.normal((H, M, D), 1410 + M + D, W.T_Q, D ** -0.5, dt, DEV)
    K = W.normal((B, H, N, D), 1410 + M + D, W.T_K, 1.0, dt, DEV)
    V = W.normal((B, H, N, D), 1410 + M + D, W.T_V, 1.0, dt, DEV)
    dZ = W.normal((B, H, M, D), 1410 + M + D, W.T_DZ, 1.0, dt, DEV)
    mask = None
    if masked:
        g = np.random.default_rng(M + D)
        m = (g.random((B, N)) > 0.3).astype(np.uint8)
        m[:, 0] = 1
        mask = torch.from_numpy(m).to(DEV)
    scale = fl.scale_for(D)
    O, Lp = fl.encode(Q, K, V, offsets, mask, scale)
    Z, L, _ = fl.lse_merge(O, Lp)
    dQ0, dK0, dV0 = fl.encode_bwd(Q, K, V, offsets, mask, scale, Z, L, dZ)
    torch.cuda.synchronize()
    e = ref.encode_ref(Q, K, V, offsets, mask, scale)
    gr = ref.encode_bwd_ref(Q, K, V, mask, scale, e["Z"], e["L"], dZ)
    if dt == torch.float32:
        for k, t in (("dQ", dQ0), ("dK", dK0), ("dV", dV0)):
            compare(t, gr[k], k, 1e-5)
    else:
        for k, t in (("dQ", dQ0), ("dK", dK0), ("dV", dV0)):
            compare_bf16(t, gr[k], k)
    prevK = torch.randn_like(dK0.float()).to(dt)
    prevV = torch.randn_like(dV0.float()).to(dt)
    inv = None if mask is None else (mask == 0)[:, None, :, None].expand_as(dK0)
    for flags in (fl.ACCUMULATE_DK, fl.ACCUMULATE_DV, fl.ACCUMULATE_DK | fl.ACCUMULATE_DV):
        dK, dV = prevK.clone(), prevV.clone()
        fl.encode_bwd(Q, K, V, offsets, mask, scale, Z, L, dZ, dK=dK, dV=dV, flags=flags)
        torch.cuda.synchronize()
        wantK = (prevK.float() + dK0.float()).to(dt) if flags & fl.ACCUMULATE_DK else dK0
        wantV = (prevV.float() + dV0.float()).to(dt) if flags & fl.ACCUMULATE_DV else dV0
        assert torch.equal(dK, wantK), flags
        assert torch.equal(dV, wantV), flags
        if inv is not None:
            if flags & fl.ACCUMULATE_DK:
                assert torch.equal(dK[inv], prevK[inv])
            if flags & fl.ACCUMULATE_DV:
                assert torch.equal(dV[inv], prevV[inv])


def test_flarepp_shared_projection_chain_small():
    """Shared projections (query-synthesis keys and values tied to K and V): forward and the
    three-call backward against the oracle's shared variant."""
    w = W.shrink(W.FLAREPP, 4000, R=4, H=2, ragged=True)
    x = w.make(DEV)
    dY = W.normal((1, 2, 4000, 64), 1510, W.T_DZ, 1.0, torch.bfloat16, DEV)
    K, V = x["K"], x["V"]
    fwd = fl.flarepp_forward(x["Qt"], K, V, K, V, w.offsets, w.scale)
    g = fl.flarepp_backward(fwd, x["Qt"], K, V, K, V, w.offsets, dY, w.scale)
    torch.cuda.synchronize()
    rf = ref.flarepp_ref(x["Qt"], K, V, K, V, w.offsets, w.scale)
    compare_bf16(fwd["Z"], rf["Z"], "Z")
    compare_bf16(fwd["Y"], rf["Y"], "Y")
    r = ref.flarepp_shared_bwd_ref(x["Qt"], K, V, w.offsets, w.scale, dY, round_qx_bf16=True)
    compare_bf16(g["dQX"], r["dQX"], "dQX")
    for k in ("dQt", "dK", "dV"):
        compare_bf16(g[k], r[k], k)
    p = ref.flarepp_shared_bwd_ref(x["Qt"], K, V, w.offsets, w.scale, dY)
    for k in ("dQX", "dQt", "dK", "dV"):
        compare_bf16(g[k], p[k], k + " plain")
    assert g["dKt"] is g["dK"] and g["dVt"] is g["dV"]


@pytest.mark.parametrize("shared", [False, True])
def test_flarepp_backward_chain_head_dim_16(shared):
    """The three-call chain at head dim 16 (the pages' C = 128, H = 8 backbone), separate or shared projections."""
    w = W.shrink(W.FLAREPP_D16, 5000, R=4, H=2, ragged=True)
    x = w.make(DEV)
    dY = W.normal((1, 2, 5000, 16), 1530, W.T_DZ, 1.0, torch.bfloat16, DEV)
    Kt, Vt = (x["K"], x["V"]) if shared else (x["Kt"], x["Vt"])
    fwd = fl.flarepp_forward(x["Qt"], Kt, Vt, x["K"], x["V"], w.offsets, w.scale)
    g = fl.flarepp_backward(fwd, x["Qt"], Kt, Vt, x["K"], x["V"], w.offsets, dY, w.scale)
    torch.cuda.synchronize()
    for rnd in (True, False):     # as executed, then the plain chain, at the same bf16 bounds
        if shared:
            r = ref.flarepp_shared_bwd_ref(x["Qt"], x["K"], x["V"], w.offsets, w.scale, dY, round_qx_bf16=rnd)
            names = ("dQt", "dK", "dV")
        else:
            r = ref.flarepp_bwd_ref(x["Qt"], x["Kt"], x["Vt"], x["K"], x["V"], w.offsets, w.scale, dY,
                                    round_qx_bf16=rnd)
            names = ("dQt", "dKt", "dVt", "dK", "dV")
        compare_bf16(g["dQX"], r["dQX"], f"dQX round={rnd}")
        for k in names:
            compare_bf16(g[k], r[k], f"{k} round={rnd}")

