"""Comparison helpers shared by the GPU parity tests."""
import numpy as np

# Tolerances: float32 inputs max-abs 1e-5; bfloat16 inputs (float32 accumulation)
# 2e-2 abs + 1e-2 rel elementwise, plus a normwise relative bound (the outputs
# at the workloads' distributions are small, which makes the absolute bound
# loose) and a bound on log-normalisers.
F32_ATOL = 1e-5
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2
BF16_NORM = 1e-2
L_ATOL_BF16 = 2e-2


def to64(t) -> np.ndarray:
    import torch
    if isinstance(t, torch.Tensor):
        t = t.detach()
        if t.dtype in (torch.bfloat16, torch.float16):
            t = t.float()
        return t.cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def compare(gpu, ref, name, atol, rtol=0.0, norm_rtol=None, report=None):
    """Elementwise |g - r| <= atol + rtol |r| with -inf matched exactly; NaN never allowed."""
    g = to64(gpu)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    keep = ~np.isnan(r)             # NaN in the reference marks "not computed"
    g, r = g[keep], r[keep]
    assert not np.isnan(g).any(), f"{name}: NaN in GPU output"
    gi, ri = np.isinf(g), np.isinf(r)
    assert np.array_equal(gi, ri) and np.array_equal(g[gi], r[ri]), f"{name}: infinities differ"
    g, r = g[~gi], r[~ri]
    if g.size == 0:
        return {"max_abs": 0.0}
    diff = np.abs(g - r)
    lim = atol + rtol * np.abs(r)
    worst = int(np.argmax(diff - lim))
    info = {"max_abs": float(diff.max()), "worst_excess": float((diff - lim)[worst])}
    nr = float(np.linalg.norm(r))
    if nr > 0:
        info["norm_rel"] = float(np.linalg.norm(g - r) / nr)
    if report is not None:
        report[name] = info
    assert (diff <= lim).all(), f"{name}: max |diff| {diff.max():.3e} (at ref {r[worst]:.4e}, gpu {g[worst]:.4e}) > tol"
    if norm_rtol is not None and nr > 0:
        assert info["norm_rel"] <= norm_rtol, f"{name}: normwise relative error {info['norm_rel']:.3e}"
    return info


def compare_bf16(gpu, ref, name, report=None):
    return compare(gpu, ref, name, BF16_ATOL, BF16_RTOL, BF16_NORM, report)


def compare_L(gpu, ref, name, fp32=False, report=None):
    return compare(gpu, ref, name, F32_ATOL if fp32 else L_ATOL_BF16, 0.0, None, report)
