"""GPU tests of the one-call encoder + merge (flare_encode_merge) and of a HIP
graph holding the FLARE++ forward chain.

The merged call must give exactly the outputs of flare_encode followed by
lse_merge (same merges in the same order), whether the merge runs inside the
encoder launch (the last workgroup of each (batch, head) folds) or the call
falls back to the two launches (vector paths, more than 256 chunks or
partitions).  It must leave its arrival counters at zero.  One case is also
checked against the oracle directly.  The graph test replays a captured
FLARE++ forward several times, with eager work and synchronisations between
the replays, and checks every replay against the eager result.
"""
import numpy as np
import pytest
import torch

import split_kv_softmax_amd as fl
import workloads as W
from oracle import flare_ref as ref
from tests._util import compare_bf16, compare_L

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(M, D, offsets, B, H, dtype=torch.bfloat16, masked=False, seed=0, q_per_batch=False):
    g = torch.Generator().manual_seed(seed)
    N = offsets[-1]
    qshape = (B, H, M, D) if q_per_batch else (H, M, D)
    Q = (torch.randn(qshape, generator=g) * D ** -0.5).to(dtype).to(DEV)
    K = torch.randn((B, H, N, D), generator=g).to(dtype).to(DEV)
    V = torch.randn((B, H, N, D), generator=g).to(dtype).to(DEV)
    mask = None
    if masked:
        m = (torch.rand((B, N), generator=g) > 0.3).to(torch.uint8)
        m[:, 0] = 1
        mask = m.to(DEV)
    return Q, K, V, mask


def _two_calls(Q, K, V, offsets, mask, scale, want_bf16):
    O_part, L_part = fl.encode(Q, K, V, offsets, mask, scale)
    Z, L, Zb = fl.lse_merge(O_part, L_part, want_bf16=want_bf16)
    return O_part, L_part, Z, L, Zb


def _assert_same(a, b, names=("O_part", "L_part", "Z", "L", "Z_bf16")):
    for x, y, n in zip(a, b, names):
        if x is None and y is None:
            continue
        assert x.shape == y.shape, n
        assert torch.equal(x, y), f"{n}: fused and two-call results differ ({(x != y).sum().item()} elements)"


CASES = {
    # merge inside the launch: pipelined encoder, ragged partitions with an empty one
    "ilv_M128_D64": dict(M=128, D=64, offsets=[0, 700, 700, 1900, 2500, 4033], B=2, H=3),
    "ilv_M64_D64": dict(M=64, D=64, offsets=[0, 1000, 1000, 3000, 3001], B=2, H=2),
    # general matrix-core encoder, padding mask, per-batch queries
    "mfma_M256_D128_masked": dict(M=256, D=128, offsets=[0, 900, 900, 2400, 3100], B=2, H=2, masked=True,
                                  q_per_batch=True),
    "mfma_M32_D64": dict(M=32, D=64, offsets=[0, 64, 129, 2000], B=1, H=4),
    # partitions split over several chunks next to a direct one and an empty one
    "split_partitions": dict(M=128, D=64, offsets=[0, 0, 30000, 30100, 40000], B=2, H=2),
    "split_partitions_masked": dict(M=64, D=128, offsets=[0, 20000, 20000, 20050, 26000], B=1, H=2, masked=True),
    # head dim 16: the general matrix-core encoder with a padding mask, and at 256 latent rows
    "mfma_M128_D16_masked": dict(M=128, D=16, offsets=[0, 700, 700, 1900, 2500, 4033], B=2, H=3, masked=True),
    "mfma_M256_D16_split": dict(M=256, D=16, offsets=[0, 20000, 20000, 20050, 26000], B=1, H=2),
    # two launches: single-query vector path, float32 vector path
    "q1_fallback": dict(M=1, D=128, offsets=[0, 5000, 5000, 9000], B=2, H=4),
    "f32_fallback": dict(M=16, D=32, offsets=[0, 300, 500, 924, 1024], B=1, H=1, dtype=torch.float32),
    # two launches: more than 256 partitions
    "many_partitions_fallback": dict(M=64, D=64, offsets=list(range(0, 300 * 40 + 1, 40)), B=1, H=2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_encode_merge_equals_encode_then_merge(name):
    c = dict(CASES[name])
    dtype = c.pop("dtype", torch.bfloat16)
    masked = c.pop("masked", False)
    qpb = c.pop("q_per_batch", False)
    M, D, offsets, B, H = c["M"], c["D"], c["offsets"], c["B"], c["H"]
    print(f"case {name}: M={M} D={D} N={offsets[-1]} R={len(offsets) - 1} B={B} H={H}", flush=True)
    Q, K, V, mask = _inputs(M, D, offsets, B, H, dtype, masked, seed=len(name), q_per_batch=qpb)
    scale = fl.scale_for(D)
    want_bf16 = dtype == torch.bfloat16
    ref_out = _two_calls(Q, K, V, offsets, mask, scale, want_bf16)
    cnt = torch.zeros(B * H * len(offsets), dtype=torch.int32, device=DEV)
    for _ in range(2):   # the second call relies on the first leaving the counters at zero
        got = fl.encode_merge(Q, K, V, offsets, mask, scale, want_bf16, counters=cnt)
        torch.cuda.synchronize()
        assert int(cnt.abs().sum()) == 0, "counters not back to zero"
        _assert_same(got, ref_out)


def test_encode_merge_chunk_count_over_one_launch_falls_back():
    # 32 latent rows at head dim 64 run three workgroups per CU, so one
    # partition of 300K tokens is cut into 300 chunks: more than one launch holds
    B, H, M, D = 1, 1, 32, 64
    offsets = [0, 300 * 1024]
    Q, K, V, _ = _inputs(M, D, offsets, B, H, seed=7)
    scale = fl.scale_for(D)
    ref_out = _two_calls(Q, K, V, offsets, None, scale, True)
    got = fl.encode_merge(Q, K, V, offsets, None, scale, True)
    torch.cuda.synchronize()
    _assert_same(got, ref_out)


def test_encode_merge_against_oracle():
    w = W.shrink(W.FLARE_BLOCK, 5000, R=6, B=2, H=2, ragged=True)
    x = w.make(DEV)
    O_part, L_part, Z, L, _ = fl.encode_merge(x["Q"], x["K"], x["V"], w.offsets, None, w.scale)
    torch.cuda.synchronize()
    e = ref.encode_ref(x["Q"], x["K"], x["V"], w.offsets, None, w.scale)
    compare_bf16(O_part, e["O_part"], "O_part")
    compare_L(L_part, e["L_part"], "L_part")
    compare_bf16(Z, e["Z"], "Z")
    compare_L(L, e["L"], "L")


def test_encode_merge_empty_token_range():
    # N = 0: every partition empty, Z = 0 and L = -inf
    B, H, M, D = 1, 2, 64, 64
    Q = torch.randn((H, M, D)).to(torch.bfloat16).to(DEV)
    K = torch.zeros((B, H, 0, D), dtype=torch.bfloat16, device=DEV)
    O_part, L_part, Z, L, Zb = fl.encode_merge(Q, K, K, [0, 0, 0], None, 0.125, True)
    torch.cuda.synchronize()
    assert torch.equal(Z, torch.zeros_like(Z)) and torch.equal(Zb.float(), torch.zeros_like(Z))
    assert bool(torch.isneginf(L).all()) and bool(torch.isneginf(L_part).all())


@pytest.mark.parametrize("fused", [False, True])
def test_flarepp_forward_graph_replays_match_eager(fused):
    w = W.shrink(W.FLAREPP, 20000, R=4, H=4, ragged=True)
    x = w.make(DEV)
    args = (x["Qt"], x["Kt"], x["Vt"], x["K"], x["V"], w.offsets, w.scale, fused)
    eager = fl.flarepp_forward(*args)   # also sizes the cached workspace and counters
    torch.cuda.synchronize()
    keys = ("QX", "QX_L", "Z", "L", "Y")
    expect = {k: eager[k].clone() for k in keys}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fl.flarepp_forward(*args)      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = fl.flarepp_forward(*args)
    for rep in range(4):
        for k in keys:
            out[k].fill_(float("nan"))     # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        for k in keys:
            assert torch.equal(out[k], expect[k]), f"replay {rep}: {k} differs from the eager result"
        other = fl.flarepp_forward(*args)   # an eager call between replays
        torch.cuda.synchronize()
        assert torch.equal(other["Y"], expect["Y"])
    assert int(fl.merge_counters(1, torch.device(DEV)).abs().sum()) == 0


@pytest.mark.parametrize("shared", [False, True])
def test_flarepp_training_step_graph_replays_match_eager(shared):
    """Forward and the three-call backward captured in one graph: every replay equals the eager step."""
    w = W.shrink(W.FLAREPP, 12000, R=4, H=2, ragged=True)
    x = w.make(DEV)
    Kt, Vt = (x["K"], x["V"]) if shared else (x["Kt"], x["Vt"])
    dY = W.normal((1, 2, 12000, 64), 1520, W.T_DZ, 1.0, torch.bfloat16, DEV)

    def step():
        fwd = fl.flarepp_forward(x["Qt"], Kt, Vt, x["K"], x["V"], w.offsets, w.scale)
        g = fl.flarepp_backward(fwd, x["Qt"], Kt, Vt, x["K"], x["V"], w.offsets, dY, w.scale)
        return fwd["Y"], g

    keys = ("dQt", "dKt", "dVt", "dK", "dV", "dQX")
    Y0, g0 = step()                      # sizes the cached workspaces outside the capture
    torch.cuda.synchronize()
    expect = {k: g0[k].clone() for k in keys}
    expect["Y"] = Y0.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        Y, g = step()
    out = dict(g)
    out["Y"] = Y
    for rep in range(3):
        for k in expect:
            out[k].zero_()               # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        for k in expect:
            assert torch.equal(out[k], expect[k]), f"replay {rep}: {k} differs from the eager step"


def test_masked_backward_graph_replays_match_eager():
    """256 latent rows at head dim 128: the backward forks its query-gradient kernel onto the
    library's second stream and joins it with events; captured in one graph with the forward,
    every replay equals the eager step, with eager calls between the replays."""
    w = W.shrink(W.MASKED_FWD_BWD, 2048, R=4, B=2, H=2)
    x = w.make(DEV)

    def step():
        O, Lp = fl.encode(x["Q"], x["K"], x["V"], w.offsets, x["mask"], w.scale)
        Z, L, _ = fl.lse_merge(O, Lp)
        return fl.encode_bwd(x["Q"], x["K"], x["V"], w.offsets, x["mask"], w.scale, Z, L, x["dZ"])

    g0 = step()                          # creates the second stream outside the capture
    torch.cuda.synchronize()
    expect = [t.clone() for t in g0]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = step()
    for rep in range(3):
        for t in out:
            t.fill_(float("nan"))        # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        for name, t, e in zip(("dQ", "dK", "dV"), out, expect):
            assert torch.equal(t, e), f"replay {rep}: {name} differs from the eager step"
        other = step()                   # an eager call between replays
        torch.cuda.synchronize()
        assert all(torch.equal(t, e) for t, e in zip(other, expect))
