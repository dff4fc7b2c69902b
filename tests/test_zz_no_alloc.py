"""flare_encode_noalloc (the encoder with the library's fixed per-device scratch in place of a
caller workspace, for callers that cannot allocate) against flare_encode on the same inputs:
the same kernels, so the states must be the same bits.  Two calls in a row, the second with
a smaller input, so the second runs over scratch the first left behind."""
import numpy as np
import pytest
import torch

import split_kv_softmax_amd as fl
import workloads as W
from oracle import flare_ref as ref
from tests._util import compare_bf16, compare_L

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(B, H, N, M, D, R, masked, wid):
    w = W.Workload(name=f"noalloc_{wid}", wid=wid, kind="encode", dtype="bf16", B=B, H=H, N=N, M=M, D=D,
                   offsets=W.ragged_offsets(N, R, wid), q_std=D ** -0.5, q_per_batch=False, stress=1.0)
    x = w.make(DEV)
    mask = None
    if masked:
        m = (np.random.default_rng(wid).random((B, N)) > 0.4).astype(np.uint8)
        m[:, 0] = 1
        mask = torch.from_numpy(m).to(DEV)
    return w, x, mask


def test_noalloc_encoder_matches_workspace_encoder_twice():
    cases = [(2, 4, 50000, 128, 64, 3, True, 3101),    # masked: mask words, launch order, split partitions
             (1, 2, 9000, 64, 64, 2, False, 3102)]     # smaller, unmasked pipelined encoder, split partitions
    for B, H, N, M, D, R, masked, wid in cases:
        print(f"noalloc case B={B} H={H} N={N} M={M} D={D} R={R} masked={masked}", flush=True)
        w, x, mask = _case(B, H, N, M, D, R, masked, wid)
        need = fl.encode_workspace_size(torch.bfloat16, B, H, N, M, D, w.offsets, masked)
        assert 0 < need <= fl.NOALLOC_SCRATCH_BYTES
        O0, L0 = fl.encode(x["Q"], x["K"], x["V"], w.offsets, mask, w.scale)
        O1 = torch.full_like(O0, float("nan"))
        L1 = torch.full_like(L0, float("nan"))
        fl.encode_noalloc(x["Q"], x["K"], x["V"], w.offsets, mask, w.scale, O1, L1)
        torch.cuda.synchronize()
        assert torch.equal(O0, O1) and torch.equal(L0, L1)
        e = ref.encode_ref(x["Q"], x["K"], x["V"], w.offsets, mask, w.scale, slices=[(0, 0), (B - 1, H - 1)])
        for b, h in ((0, 0), (B - 1, H - 1)):
            compare_bf16(O1[:, b, h], e["O_part"][:, b, h], f"O_part[{b},{h}]")
            compare_L(L1[:, b, h], e["L_part"][:, b, h], f"L_part[{b},{h}]")


def test_noalloc_encoder_rejects_beyond_its_scratch():
    """Arguments whose workspace exceeds the fixed scratch: FLARE_EWORKSPACE, outputs untouched."""
    N = 1 << 20
    K = torch.zeros((1, 1, N, 128), dtype=torch.bfloat16, device=DEV)
    Q = torch.zeros((1, 256, 128), dtype=torch.bfloat16, device=DEV)
    O = torch.full((1, 1, 1, 256, 128), 7.0, device=DEV)
    L = torch.full((1, 1, 1, 256), 7.0, device=DEV)
    with pytest.raises(fl.FlareError) as ei:
        fl.encode_noalloc(Q, K, K, [0, N], None, None, O, L)
    assert ei.value.status == -4 and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert (O == 7).all() and (L == 7).all()
