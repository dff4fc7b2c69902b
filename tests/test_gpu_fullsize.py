"""Parity at the workloads' full sizes, in the launch configuration the benchmark times.

The whole path runs on the GPU at full size.  The float64 oracle then
recomputes a sample of (batch, head) slices one by one from the very same
input bits (and, for the decodes, a sample of token rows), and properties that
hold at any size are checked on every output: finite values, exact empty
partitions, zero gradient rows for padding.
"""
import os
import sys

import numpy as np
import pytest
import torch

import split_kv_softmax_amd as fl
import workloads as W
from oracle import flare_ref as ref
from tests._util import F32_ATOL, compare, compare_bf16, compare_L

pytestmark = pytest.mark.gpu
DEV = "cuda"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _say(msg):
    print(msg, flush=True)


def _host_slice(t, b, h, q_per_batch=True):
    """[1, 1, ...] host copy of slice (b, h) of a [B, H, ...] tensor ([1, ...] for replicated Q)."""
    if t.dim() == 3:                   # replicated [H, M, D]
        return t[h:h + 1].cpu()
    return t[b:b + 1, h:h + 1].cpu()


def _finite(t, name):
    assert bool(torch.isfinite(t).all()), f"{name}: non-finite values"


def _sample_tokens(N, k, seed):
    return np.sort(np.random.default_rng(seed).choice(N, size=min(k, N), replace=False))


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_full_fp32_small_encoder():
    w = W.FLARE_ENCODE_F32_SMALL
    _say(f"case {w.name}")
    x = w.make(DEV)
    O, Lp = fl.encode(x["Q"], x["K"], x["V"], w.offsets, None, w.scale)
    Z, L, _ = fl.lse_merge(O, Lp)
    torch.cuda.synchronize()
    e = ref.encode_ref(x["Q"], x["K"], x["V"], w.offsets, None, w.scale)
    for g, k in ((O, "O_part"), (Lp, "L_part"), (Z, "Z"), (L, "L")):
        compare(g, e[k], k, F32_ATOL)


def test_full_flare_block():
    """FLARE block at B=2, H=8, N=65536, M=64, D=64, R=8: encode, merge, decode."""
    w = W.FLARE_BLOCK
    _say(f"case {w.name}")
    x = w.make(DEV)
    out = fl.flare_forward(x["Q"], x["K"], x["V"], w.offsets, None, w.scale)
    torch.cuda.synchronize()
    for k in ("O_part", "L_part", "Z", "L", "Y"):
        _finite(out[k], k)
    for b, h in ((0, 0), (1, 5), (0, 7)):
        q = _host_slice(x["Q"], b, h)
        k_, v_ = _host_slice(x["K"], b, h), _host_slice(x["V"], b, h)
        e = ref.encode_ref(q, k_, v_, w.offsets, None, w.scale)
        compare_bf16(out["O_part"][:, b:b + 1, h:h + 1], e["O_part"], f"O_part[{b},{h}]")
        compare_L(out["L_part"][:, b:b + 1, h:h + 1], e["L_part"], f"L_part[{b},{h}]")
        compare_bf16(out["Z"][b:b + 1, h:h + 1], e["Z"], f"Z[{b},{h}]")
        compare_L(out["L"][b:b + 1, h:h + 1], e["L"], f"L[{b},{h}]")
        idx = _sample_tokens(w.N, 4096, 11 + b * 8 + h)
        y = ref.decode_ref(k_[:, :, idx], q, e["Z"], w.scale)
        compare_bf16(out["Y"][b:b + 1, h:h + 1, idx], y, f"Y[{b},{h}] sampled")


def test_full_flarepp_chain_as_benchmarked():
    """FLARE++ at B=1, H=16, N=262144, M=128, D=64, R=16, through the benchmark's own step."""
    sys.path.insert(0, ROOT)
    import bench
    w = W.FLAREPP
    _say(f"case {w.name}")
    x = w.make(DEV)
    step = bench.FlareppStep(w, x)
    step()
    torch.cuda.synchronize()
    for name in ("O1", "L1", "QX", "QXL", "O2", "L2", "Z", "L", "Y"):
        _finite(getattr(step, name), name)
    assert torch.equal(step.QXb, step.QX.to(torch.bfloat16))
    for h in (0, 11):
        xs = {k: v[:, h:h + 1].cpu() if v.dim() == 4 else v[h:h + 1].cpu() for k, v in x.items()}
        r = ref.flarepp_ref(xs["Qt"], xs["Kt"], xs["Vt"], xs["K"], xs["V"], w.offsets, w.scale)
        compare_bf16(step.QX[:, h:h + 1], r["QX"], f"QX[h={h}]")
        compare_bf16(step.O2[:, :, h:h + 1], r["O_part"], f"O_part[h={h}]")
        compare_L(step.L2[:, :, h:h + 1], r["L_part"], f"L_part[h={h}]")
        compare_bf16(step.Z[:, h:h + 1], r["Z"], f"Z[h={h}]")
        compare_L(step.L[:, h:h + 1], r["L"], f"L[h={h}]")
        compare_bf16(step.Y[:, h:h + 1], r["Y"], f"Y[h={h}]")


@pytest.mark.parametrize("fused,shared", [(False, False), (True, True)])
def test_full_flarepp_head_dim_16(fused, shared):
    """FLARE++ at head dim 16 (B=1, H=8, N=2^20, M=128, R=16) through the benchmark's step, also with
    the one-call encoder + merge and the shared projections; two heads against the oracle."""
    sys.path.insert(0, ROOT)
    import bench
    w = W.FLAREPP_D16
    _say(f"case {w.name} fused={fused} shared={shared}")
    x = w.make(DEV)
    step = bench.FlareppStep(w, x, fused, shared)
    step()
    torch.cuda.synchronize()
    for name in ("O1", "L1", "QX", "QXL", "O2", "L2", "Z", "L", "Y"):
        _finite(getattr(step, name), name)
    assert torch.equal(step.QXb, step.QX.to(torch.bfloat16))
    for h in (0, 5):
        xs = {k: v[:, h:h + 1].cpu() if v.dim() == 4 else v[h:h + 1].cpu() for k, v in x.items()}
        kt, vt = (xs["K"], xs["V"]) if shared else (xs["Kt"], xs["Vt"])
        r = ref.flarepp_ref(xs["Qt"], kt, vt, xs["K"], xs["V"], w.offsets, w.scale)
        compare_bf16(step.QX[:, h:h + 1], r["QX"], f"QX[h={h}]")
        compare_bf16(step.O2[:, :, h:h + 1], r["O_part"], f"O_part[h={h}]")
        compare_L(step.L2[:, :, h:h + 1], r["L_part"], f"L_part[h={h}]")
        compare_bf16(step.Z[:, h:h + 1], r["Z"], f"Z[h={h}]")
        compare_L(step.L[:, h:h + 1], r["L"], f"L[h={h}]")
        compare_bf16(step.Y[:, h:h + 1], r["Y"], f"Y[h={h}]")


def test_full_single_query_split_kv():
    """Single-query split-KV at B=8, H=32, N=131072, D=128, P=64: encode + 6-round tree."""
    w = W.SPLITKV_Q1
    _say(f"case {w.name}")
    x = w.make(DEV)
    O, Lp = fl.encode(x["Q"], x["K"], x["V"], w.offsets, None, w.scale)
    Z, L, _ = fl.lse_merge(O, Lp)
    torch.cuda.synchronize()
    for t, k in ((O, "O_part"), (Lp, "L_part"), (Z, "Z"), (L, "L")):
        _finite(t, k)
    for b, h in ((0, 0), (3, 17), (7, 31), (5, 2)):
        q = _host_slice(x["Q"], b, h)
        e = ref.encode_ref(q, _host_slice(x["K"], b, h), _host_slice(x["V"], b, h), w.offsets, None, w.scale)
        compare_bf16(O[:, b:b + 1, h:h + 1], e["O_part"], f"O_part[{b},{h}]")
        compare_L(Lp[:, b:b + 1, h:h + 1], e["L_part"], f"L_part[{b},{h}]")
        compare_bf16(Z[b:b + 1, h:h + 1], e["Z"], f"Z[{b},{h}]")
        compare_L(L[b:b + 1, h:h + 1], e["L"], f"L[{b},{h}]")


def test_full_masked_ragged_forward_backward():
    """Masked ragged encoder at B=4, H=8, N=262144, M=256, D=128, R=16: forward and backward."""
    w = W.MASKED_FWD_BWD
    _say(f"case {w.name}")
    x = w.make(DEV)
    lens, _ = W.prefix_lengths_mask(w.B, w.R, w.mask_slot, w.wid)
    O, Lp = fl.encode(x["Q"], x["K"], x["V"], w.offsets, x["mask"], w.scale)
    Z, L, _ = fl.lse_merge(O, Lp)
    dQ, dK, dV = fl.encode_bwd(x["Q"], x["K"], x["V"], w.offsets, x["mask"], w.scale, Z, L, x["dZ"])
    torch.cuda.synchronize()
    for t, k in ((O, "O_part"), (Z, "Z"), (L, "L"), (dQ, "dQ"), (dK, "dK"), (dV, "dV")):
        _finite(t, k)
    # empty partitions: exactly (-inf, 0); padding rows: exactly zero gradients
    empty = [(b, r) for b in range(w.B) for r in range(w.R) if lens[b, r] == 0]
    assert empty, "the workload has a fully empty partition"
    for b, r in empty:
        assert bool((Lp[r, b] == float("-inf")).all()) and bool((O[r, b] == 0).all())
    for b in range(w.B):
        pad = x["mask"][b] == 0
        assert bool((dK[b][:, pad] == 0).all()) and bool((dV[b][:, pad] == 0).all())
    b_star = empty[0][0]
    for b, h in ((b_star, 0), ((b_star + 1) % w.B, 5)):
        q, k_, v_ = _host_slice(x["Q"], b, h), _host_slice(x["K"], b, h), _host_slice(x["V"], b, h)
        m_ = x["mask"][b:b + 1].cpu()
        e = ref.encode_ref(q, k_, v_, w.offsets, m_, w.scale)
        compare_bf16(O[:, b:b + 1, h:h + 1], e["O_part"], f"O_part[{b},{h}]")
        compare_L(Lp[:, b:b + 1, h:h + 1], e["L_part"], f"L_part[{b},{h}]")
        compare_bf16(Z[b:b + 1, h:h + 1], e["Z"], f"Z[{b},{h}]")
        compare_L(L[b:b + 1, h:h + 1], e["L"], f"L[{b},{h}]")
        dz = _host_slice(x["dZ"], b, h)
        g = ref.encode_bwd_ref(q, k_, v_, m_, w.scale, Z[b:b + 1, h:h + 1].cpu(), L[b:b + 1, h:h + 1].cpu(), dz)
        compare_bf16(dQ[b:b + 1, h:h + 1], g["dQ"], f"dQ[{b},{h}]")
        compare_bf16(dK[b:b + 1, h:h + 1], g["dK"], f"dK[{b},{h}]")
        compare_bf16(dV[b:b + 1, h:h + 1], g["dV"], f"dV[{b},{h}]")


def test_full_flarepp_backward_chain():
    """FLARE++ backward chain at B=1, H=16, N=262144, M=128, D=64, R=16 (decoder, physical-value
    encoder, query-synthesis encoder); two heads recomputed by the oracle as executed
    (Q(X) rounded to bf16), every output checked finite."""
    w = W.FLAREPP
    _say(f"case {w.name} backward")
    x = w.make(DEV)
    dY = W.normal((w.B, w.H, w.N, w.D), w.wid, W.T_DZ, 1.0, torch.bfloat16, DEV)
    fwd = fl.flarepp_forward(x["Qt"], x["Kt"], x["Vt"], x["K"], x["V"], w.offsets, w.scale)
    g = fl.flarepp_backward(fwd, x["Qt"], x["Kt"], x["Vt"], x["K"], x["V"], w.offsets, dY, w.scale)
    torch.cuda.synchronize()
    for k, t in g.items():
        _finite(t, k)
    for h in (3, 12):
        xs = {k: v[:, h:h + 1].cpu() if v.dim() == 4 else v[h:h + 1].cpu() for k, v in x.items()}
        r = ref.flarepp_bwd_ref(xs["Qt"], xs["Kt"], xs["Vt"], xs["K"], xs["V"], w.offsets, w.scale,
                                dY[:, h:h + 1].cpu(), round_qx_bf16=True)
        compare_bf16(g["dQX"][:, h:h + 1], r["dQX"], f"dQX[h={h}]")
        for k in ("dQt", "dKt", "dVt", "dK", "dV"):
            compare_bf16(g[k][:, h:h + 1], r[k], f"{k}[h={h}]")
    # the plain chain (Q(X) kept in float64) on one head, at the same bf16 bounds
    h = 3
    xs = {k: v[:, h:h + 1].cpu() if v.dim() == 4 else v[h:h + 1].cpu() for k, v in x.items()}
    p = ref.flarepp_bwd_ref(xs["Qt"], xs["Kt"], xs["Vt"], xs["K"], xs["V"], w.offsets, w.scale,
                            dY[:, h:h + 1].cpu())
    for k in ("dQX", "dQt", "dKt", "dVt", "dK", "dV"):
        compare_bf16(g[k][:, h:h + 1], p[k], f"{k}[h={h}] plain")


def test_full_flarepp_backward_chain_head_dim_16():
    """FLARE++ backward chain at head dim 16 (B=1, H=8, N=2^20, M=128, R=16), every output finite, one
    head recomputed by the oracle as executed (Q(X) rounded to bf16)."""
    w = W.FLAREPP_D16
    _say(f"case {w.name} backward")
    x = w.make(DEV)
    dY = W.normal((w.B, w.H, w.N, w.D), w.wid, W.T_DZ, 1.0, torch.bfloat16, DEV)
    fwd = fl.flarepp_forward(x["Qt"], x["Kt"], x["Vt"], x["K"], x["V"], w.offsets, w.scale)
    g = fl.flarepp_backward(fwd, x["Qt"], x["Kt"], x["Vt"], x["K"], x["V"], w.offsets, dY, w.scale)
    torch.cuda.synchronize()
    for k, t in g.items():
        _finite(t, k)
    h = 6
    xs = {k: v[:, h:h + 1].cpu() if v.dim() == 4 else v[h:h + 1].cpu() for k, v in x.items()}
    r = ref.flarepp_bwd_ref(xs["Qt"], xs["Kt"], xs["Vt"], xs["K"], xs["V"], w.offsets, w.scale,
                            dY[:, h:h + 1].cpu(), round_qx_bf16=True)
    compare_bf16(g["dQX"][:, h:h + 1], r["dQX"], f"dQX[h={h}]")
    for k in ("dQt", "dKt", "dVt", "dK", "dV"):
        compare_bf16(g[k][:, h:h + 1], r[k], f"{k}[h={h}]")
    p = ref.flarepp_bwd_ref(xs["Qt"], xs["Kt"], xs["Vt"], xs["K"], xs["V"], w.offsets, w.scale,
                            dY[:, h:h + 1].cpu())
    for k in ("dQX", "dQt", "dKt", "dVt", "dK", "dV"):
        compare_bf16(g[k][:, h:h + 1], p[k], f"{k}[h={h}] plain")

