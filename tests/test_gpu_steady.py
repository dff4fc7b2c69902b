"""GPU parity of the encoder's steady rounds and the decode's steady blocks.

The pipelined encoder and the matrix-core decode run most of a long chunk or
token run in a steady form (fixed ring waits, loads without row checks, no
bounds tests) and fall back to the general form for the ring's fill and tail.
The small parity cases of the other files never reach the steady form, so the
cases here use chunks and runs long enough for several steady trips, with
ragged tails, re-bases of the softmax reference inside the steady rounds,
masked tokens and padded NaN rows inside steady blocks, and tokens that take
the decode's exact form.  Every output is compared with the float64 oracle.
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

# partition lengths 5000, 0, 8333, 7667: the library splits them into chunks of
# at most 4096 tokens (a 4096-token chunk is 32 tiles per token group, 26 of
# them in steady rounds) and the chunk tails end in partial tiles
OFFS = [0, 5000, 5000, 13333, 21000]


def _encoder_case(M, D, wid, stress=1.0):
    N = OFFS[-1]
    w = W.Workload(name=f"steady_M{M}_D{D}", wid=wid, kind="encode", dtype="bf16", B=1, H=2, N=N, M=M, D=D,
                   offsets=OFFS, q_std=D ** -0.5, q_per_batch=False, stress=stress)
    return w, w.make(DEV)


def _check(w, x, Q=None, K=None, scale=None):
    Q = x["Q"] if Q is None else Q
    K = x["K"] if K is None else K
    sc = w.scale if scale is None else scale
    O_part, L_part = fl.encode(Q, K, x["V"], w.offsets, None, sc)
    Z, L, _ = fl.lse_merge(O_part, L_part)
    torch.cuda.synchronize()
    out = ref.encode_ref(Q, K, x["V"], w.offsets, None, sc)
    compare_bf16(O_part, out["O_part"], "O_part")
    compare_L(L_part, out["L_part"], "L_part")
    compare_bf16(Z, out["Z"], "Z")
    compare_L(L, out["L"], "L")
    return L


@pytest.mark.parametrize("M,D", [(128, 64), (64, 64), (128, 16), (64, 16)])
def test_encoder_steady_rounds_ragged_chunks(M, D):
    """Chunks of up to 4096 tokens (several steady trips) and ragged chunk tails."""
    w, x = _encoder_case(M, D, 900 + M + D)
    assert fl.encode_workspace_size(torch.bfloat16, 1, 2, w.N, M, D, w.offsets) > 0, "partitions are split"
    _check(w, x)


@pytest.mark.parametrize("M,D", [(128, 64), (128, 16)])
def test_encoder_rebases_inside_steady_rounds(M, D):
    """A score spread of ~4 natural units per row over the run, so the lazily held
    reference keeps moving up inside the steady rounds; plus rows whose scores grow
    along the sequence (keys scaled up by position), which re-base late in the chunk."""
    w, x = _encoder_case(M, D, 950 + M + D, stress=4 * 8.0)
    _check(w, x)
    K = x["K"].float().clone()
    ramp = torch.linspace(0.5, 3.0, w.N, device=DEV).view(1, 1, w.N, 1)
    K = (K * ramp).to(torch.bfloat16)
    _check(w, x, K=K)


def test_encoder_far_negative_rows_in_steady_rounds():
    """Rows whose every score sits near -300 (weights against a zero reference
    underflow; head dim 16 re-bases downwards) over long chunks."""
    M, D = 128, 16
    w, x = _encoder_case(M, D, 990)
    Q = x["Q"].float().clone()
    K = x["K"].float().clone()
    c = 12.0
    K[..., 0] = c
    Q[:, : M // 4, :] = 0.0
    Q[:, : M // 4, 0] = -c
    sc = float(np.float32(300.0 / (c * c)))
    L = _check(w, x, Q=Q.to(torch.bfloat16), K=K.to(torch.bfloat16), scale=sc)
    assert float(L[0, 0, 0]) < -250.0


def _decode_case(M, D, wid, N):
    B, H = 2, 8
    Xq = W.normal((B, H, N, D), wid, W.T_K, 1.0, torch.bfloat16, DEV)
    Kl = W.normal((H, M, D), wid, W.T_Q, 1.0, torch.bfloat16, DEV)
    Z = W.normal((B, H, M, D), wid, W.T_V, 1.0, torch.float32, DEV)
    return Xq, Kl, Z


@pytest.mark.parametrize("M,D", [(128, 64), (64, 64), (128, 16)])
def test_decode_steady_blocks_ragged_run(M, D):
    """16 (batch, head) slices of 65613 tokens: runs of 2304 tokens per workgroup,
    nine 32-token blocks per wave (one steady trip), the last run ragged."""
    N = 65613
    Xq, Kl, Z = _decode_case(M, D, 960 + M + D, N)
    s = W.scale_for(D)
    Y = fl.decode(Xq, Kl, Z, s)
    torch.cuda.synchronize()
    compare_bf16(Y, ref.decode_ref(Xq, Kl, Z, s), "Y")


def test_decode_steady_blocks_masks_nan_rows_and_exact_form():
    """Masked tokens (zeros out, NaN rows at some of them) and tokens whose row
    sums overflow the zero reference (exact form) inside steady blocks."""
    M, D, N = 128, 64, 65613
    Xq, Kl, Z = _decode_case(M, D, 977, N)
    g = torch.Generator().manual_seed(5)
    tm = (torch.rand(2, N, generator=g) > 0.1).to(torch.uint8)
    tm[1, 20000:20400] = 0
    hot = torch.randint(0, N, (400,), generator=g)
    Xh = Xq.float()
    Xh[:, :, hot] *= 40.0                      # scores far above the zero reference
    nan_at = torch.nonzero(tm[0] == 0).flatten()[:50]
    Xh[0, :, nan_at] = float("nan")            # padded rows may hold anything
    Xq = Xh.to(torch.bfloat16)
    tm = tm.to(DEV)
    s = W.scale_for(D)
    Y = fl.decode(Xq, Kl, Z, s, token_mask=tm)
    torch.cuda.synchronize()
    Yr = ref.decode_ref(Xq.nan_to_num(0.0), Kl, Z, s, token_mask=tm)
    compare_bf16(Y, Yr, "Y")
    assert torch.equal(Y[0, :, nan_at], torch.zeros_like(Y[0, :, nan_at]))


# ---- the pipelined encoder at head dim 128, 256 latent rows, padding masks
def _masked128_case(N, offs, mask, wid, B=2, H=2):
    M, D = 256, 128
    w = W.Workload(name=f"masked128_{wid}", wid=wid, kind="encode", dtype="bf16", B=B, H=H, N=N, M=M, D=D,
                   offsets=offs, q_std=D ** -0.5, q_per_batch=False)
    x = w.make(DEV)
    x["mask"] = torch.from_numpy(mask).to(DEV)
    return w, x


def _check_masked(w, x):
    O_part, L_part = fl.encode(x["Q"], x["K"], x["V"], w.offsets, x["mask"], w.scale)
    Z, L, _ = fl.lse_merge(O_part, L_part)
    torch.cuda.synchronize()
    out = ref.encode_ref(x["Q"], x["K"], x["V"], w.offsets, x["mask"], w.scale)
    compare_bf16(O_part, out["O_part"], "O_part")
    compare_L(L_part, out["L_part"], "L_part")
    compare_bf16(Z, out["Z"], "Z")
    compare_L(L, out["L"], "L")


def test_masked_head_dim_128_prefix_edges():
    """Valid prefixes (each chunk then runs as unmasked over its prefix) with the
    edge cases of the chunk-end scan: empty prefixes, one valid token, fully
    valid partitions, partitions and prefix ends at various offsets within and
    across 64-token mask words; plus NaN in the padded K and V rows."""
    offs = [0, 1000, 2531, 4000, 4100, 6000, 7777, 9000]
    lens = [[0, 1, 64 * 5, 65, 100, 1900, 1, 1223], [999, 1531, 1469, 100, 1, 0, 1777, 17]]
    N = offs[-1]
    mask = np.zeros((2, N), dtype=np.uint8)
    for b in range(2):
        for r in range(len(offs) - 1):
            mask[b, offs[r]: offs[r] + min(lens[b][r], offs[r + 1] - offs[r])] = 1
    w, x = _masked128_case(N, offs, mask, 1201)
    pad = torch.from_numpy(mask == 0).to(DEV)
    for t in ("K", "V"):
        v = x[t].float()
        v[:, :, :, 0][pad.view(2, 1, N).expand(2, 2, N)] = float("nan")
        x[t] = v.to(torch.bfloat16)
    _check_masked(w, x)


def test_masked_head_dim_128_holes_and_split_chunks():
    """Masks with holes inside the valid range (the chunk runs masked: every tile
    masks its scores and zeroes its invalid V rows), NaN padding, and partitions
    long enough to be split into chunks of 8192 tokens (one (batch, head) slice
    and three partitions)."""
    offs = [0, 20000, 20001, 45000]
    N = offs[-1]
    g = np.random.default_rng(1202)
    mask = (g.random((1, N)) > 0.3).astype(np.uint8)
    mask[0, 30000:30100] = 0
    mask[0, 44000:] = 0
    w, x = _masked128_case(N, offs, mask, 1202, B=1, H=1)
    pad = torch.from_numpy(mask == 0).to(DEV)
    v = x["V"].float()
    v[:, :, :, 3][pad.view(1, 1, N)] = float("nan")
    x["V"] = v.to(torch.bfloat16)
    _check_masked(w, x)
