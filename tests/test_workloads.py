"""The seeded input recipe (CPU only): shapes, determinism and the masked-workload structure."""
import numpy as np
import torch

import workloads as W


def test_draws_are_deterministic_and_rounded():
    a = W.normal((2, 3, 5), 9, W.T_K, 0.125, torch.bfloat16)
    b = W.normal((2, 3, 5), 9, W.T_K, 0.125, torch.bfloat16)
    assert torch.equal(a, b) and a.dtype == torch.bfloat16
    c = W.normal((2, 3, 5), 9, W.T_V, 0.125, torch.bfloat16)
    assert not torch.equal(a, c)


def test_masked_recipe_has_empty_partition_and_no_empty_batch():
    w = W.MASKED_FWD_BWD
    lens, mask = W.prefix_lengths_mask(w.B, w.R, w.mask_slot, w.wid)
    assert lens.shape == (w.B, w.R) and mask.shape == (w.B, w.N)
    assert (lens >= 0).all() and (lens <= w.mask_slot).all()
    assert (lens == 0).any()
    assert (lens.sum(1) > 0).all()
    for b in range(w.B):
        for r in range(w.R):
            seg = mask[b, r * w.mask_slot:(r + 1) * w.mask_slot]
            assert seg[:lens[b, r]].all() and not seg[lens[b, r]:].any()


def test_workload_shapes_and_offsets():
    for w in W.ALL + W.EXTRA:
        assert w.offsets[0] == 0 and w.offsets[-1] == w.N
        assert all(a <= b for a, b in zip(w.offsets, w.offsets[1:]))
    s = W.shrink(W.FLAREPP, 3000, R=5, ragged=True)
    x = s.make()
    assert x["Kt"].shape == (1, 16, 3000, 64) and x["Qt"].shape == (16, 128, 64)
    assert W.FLARE_ENCODE_F32_SMALL.offsets == [0, 300, 500, 924, 1024]
    assert W.scale_for(64) == 0.125
