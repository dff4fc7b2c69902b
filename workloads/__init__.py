"""Seeded synthetic inputs for the split-KV / FLARE softmax path.

This module draws random tensors, partition offsets and padding masks and
nothing else: it holds none of the method's arithmetic, so both the HIP path
and the CPU oracle can take their inputs from it without sharing any of the
computation.  Tests hand the very same tensors (bit for bit) to both sides:
the oracle widens whatever bits were sent to the device.

Recipe (every tensor): ``torch.randn`` in float32 from a generator seeded by a
64-bit key derived from ``(SEED, workload id, tensor id)`` with numpy's
``SeedSequence``, multiplied by the tensor's standard deviation in float32,
then rounded to the compute dtype (round-to-nearest-even for bfloat16).  Large
tensors are drawn directly on the device they are used on, one batch slice at
a time, so host memory stays small.

The workloads follow the FLARE++ appendix ("FLARE++: Low-rank attention with
dynamic attention routing", context-parallel encoder section): a replicated
latent query tensor of shape H x M x D, token-sharded keys and values, and
unequal shards whose padding is excluded by a mask.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch

SEED = 20261202

# tensor ids used in the seed key
T_Q, T_K, T_V, T_QT, T_KT, T_VT, T_DZ, T_LEN = range(8)


def _key(workload_id: int, tensor_id: int, extra: int = 0) -> int:
    ss = np.random.SeedSequence([SEED, workload_id, tensor_id, extra])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def normal(shape, workload_id: int, tensor_id: int, std: float, dtype: torch.dtype,
           device="cpu") -> torch.Tensor:
    """N(0, std^2) draws rounded to ``dtype``; batch slices seeded separately."""
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=dtype, device=device)
    lead = shape[0] if len(shape) > 1 else 1
    view = out.view(lead, -1) if len(shape) > 1 else out.view(1, -1)
    std32 = torch.tensor(std, dtype=torch.float32).item()
    for b in range(lead):
        g = torch.Generator(device=device)
        g.manual_seed(_key(workload_id, tensor_id, b))
        x = torch.randn(view.shape[1], generator=g, device=device, dtype=torch.float32)
        if std32 != 1.0:
            x.mul_(std32)
        view[b].copy_(x.to(dtype))
        del x
    return out


def scale_for(D: int) -> float:
    """s = D^-1/2 as the float32 value that the kernels receive."""
    return float(np.float32(1.0) / np.sqrt(np.float32(D)))


def equal_offsets(N: int, R: int) -> List[int]:
    return [N * r // R for r in range(R + 1)]


def ragged_offsets(N: int, R: int, workload_id: int) -> List[int]:
    """R partitions of random unequal length (some may be empty) covering [0, N)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, workload_id, T_LEN, 1])))
    cuts = np.sort(rng.integers(0, N + 1, size=R - 1))
    return [0] + [int(c) for c in cuts] + [N]


def prefix_lengths_mask(B: int, R: int, slot: int, workload_id: int,
                        force_empty: bool = True) -> (np.ndarray, np.ndarray):
    """Per-batch valid prefix lengths ``len[b, r] ~ U{0..slot}`` inside fixed slots.

    Partition r of batch b covers slot ``[r*slot, (r+1)*slot)``; its first
    ``len[b, r]`` tokens are valid and the rest is padding.  When no length of
    zero was drawn, one seeded (b, r) pair is set to zero so that some
    partition is fully empty; a batch whose lengths are all zero is redrawn,
    so every attention row keeps at least one valid key globally.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, workload_id, T_LEN, 0])))
    lens = rng.integers(0, slot + 1, size=(B, R))
    for b in range(B):
        while lens[b].sum() == 0:
            lens[b] = rng.integers(0, slot + 1, size=R)
    if force_empty and R >= 2 and not (lens == 0).any():
        # every length is positive here, so zeroing one keeps its batch non-empty
        b_star = int(rng.integers(0, B))
        r_star = int(rng.integers(0, R))
        lens[b_star, r_star] = 0
    mask = np.zeros((B, R * slot), dtype=np.uint8)
    for b in range(B):
        for r in range(R):
            mask[b, r * slot: r * slot + lens[b, r]] = 1
    return lens, mask


@dataclasses.dataclass
class Workload:
    """One synthetic problem: shapes, dtype, partitioning and distributions."""
    name: str
    wid: int
    kind: str            # "encode", "flare", "flarepp", "splitkv", "encode_bwd"
    dtype: str           # "f32" or "bf16"
    B: int
    H: int
    N: int
    M: int
    D: int
    offsets: List[int]
    q_std: float
    q_per_batch: bool    # Q is [B,H,M,D] (else replicated [H,M,D])
    masked: bool = False
    mask_slot: int = 0
    stress: float = 1.0  # extra factor on Q (score spread), 1 = the stated distribution

    @property
    def R(self) -> int:
        return len(self.offsets) - 1

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def scale(self) -> float:
        return scale_for(self.D)

    @property
    def tokens(self) -> int:
        return self.B * self.N * self.H

    def describe(self) -> Dict:
        return {"workload": self.name, "kind": self.kind, "dtype": self.dtype, "B": self.B,
                "H": self.H, "N": self.N, "M": self.M, "D": self.D, "R": self.R}

    def make(self, device="cpu") -> Dict[str, torch.Tensor]:
        """Draw every input of this workload on ``device``."""
        dt = self.torch_dtype
        B, H, N, M, D = self.B, self.H, self.N, self.M, self.D
        qs = self.q_std * self.stress
        out: Dict[str, torch.Tensor] = {}
        qshape = (B, H, M, D) if self.q_per_batch else (H, M, D)
        if self.kind == "flarepp":
            out["Qt"] = normal(qshape, self.wid, T_QT, qs, dt, device)
            out["Kt"] = normal((B, H, N, D), self.wid, T_KT, 1.0, dt, device)
            out["Vt"] = normal((B, H, N, D), self.wid, T_VT, 1.0, dt, device)
        else:
            out["Q"] = normal(qshape, self.wid, T_Q, qs, dt, device)
        out["K"] = normal((B, H, N, D), self.wid, T_K, 1.0, dt, device)
        out["V"] = normal((B, H, N, D), self.wid, T_V, 1.0, dt, device)
        if self.masked:
            _, mask = prefix_lengths_mask(B, self.R, self.mask_slot, self.wid)
            out["mask"] = torch.from_numpy(mask).to(device)
        if self.kind == "encode_bwd":
            out["dZ"] = normal((B, H, M, D), self.wid, T_DZ, 1.0, dt, device)
        return out

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _w(**kw) -> Workload:
    return Workload(**kw)


# The five workloads, named by what they are.
FLARE_ENCODE_F32_SMALL = _w(
    name="flare_encode_fp32_B1_H1_N1024_M16_D32_R4", wid=1, kind="encode", dtype="f32",
    B=1, H=1, N=1024, M=16, D=32, offsets=[0, 300, 500, 924, 1024], q_std=1.0, q_per_batch=True)
FLARE_BLOCK = _w(
    name="flare_block_bf16_B2_H8_N65536_M64_D64_R8", wid=2, kind="flare", dtype="bf16",
    B=2, H=8, N=65536, M=64, D=64, offsets=equal_offsets(65536, 8), q_std=1 / 8.0, q_per_batch=False)
FLAREPP = _w(
    name="flarepp_fwd_bf16_B1_H16_N262144_M128_D64_R16", wid=3, kind="flarepp", dtype="bf16",
    B=1, H=16, N=262144, M=128, D=64, offsets=equal_offsets(262144, 16), q_std=1 / 8.0,
    q_per_batch=False)
SPLITKV_Q1 = _w(
    name="splitkv_single_query_bf16_B8_H32_N131072_M1_D128_P64", wid=4, kind="splitkv",
    dtype="bf16", B=8, H=32, N=131072, M=1, D=128, offsets=equal_offsets(131072, 64),
    q_std=float(1 / np.sqrt(128.0)), q_per_batch=True)
MASKED_FWD_BWD = _w(
    name="masked_ragged_encode_fwd_bwd_bf16_B4_H8_N262144_M256_D128_R16", wid=5,
    kind="encode_bwd", dtype="bf16", B=4, H=8, N=262144, M=256, D=128,
    offsets=equal_offsets(262144, 16), q_std=float(1 / np.sqrt(128.0)), q_per_batch=False,
    masked=True, mask_slot=16384)

ALL = [FLARE_ENCODE_F32_SMALL, FLARE_BLOCK, FLAREPP, SPLITKV_Q1, MASKED_FWD_BWD]

# Beyond the five: the FLARE++ chain at the head dim of the pages' step-time
# sweep (a C = 128 backbone with H = 8 heads, so D = 16), at its largest token
# count (about 10^6, here 2^20) and the latent count of the FLARE++ workload
# above (the sweep's own M is not stated).
FLAREPP_D16 = _w(
    name="flarepp_fwd_bf16_B1_H8_N1048576_M128_D16_R16", wid=6, kind="flarepp", dtype="bf16",
    B=1, H=8, N=1048576, M=128, D=16, offsets=equal_offsets(1048576, 16), q_std=0.25,
    q_per_batch=False)
EXTRA = [FLAREPP_D16]
BY_NAME = {w.name: w for w in ALL + EXTRA}


def shrink(w: Workload, N: int, R: Optional[int] = None, B: Optional[int] = None,
           H: Optional[int] = None, ragged: bool = False, wid_offset: int = 100) -> Workload:
    """A smaller copy of a workload (same M, D, dtype, distributions) for oracle-sized parity."""
    R = R if R is not None else w.R
    B = B if B is not None else w.B
    H = H if H is not None else w.H
    kw = dict(name=f"{w.name}__N{N}_R{R}_B{B}_H{H}{'_ragged' if ragged else ''}",
              wid=w.wid + wid_offset, N=N, B=B, H=H)
    if w.masked:
        slot = N // R
        kw.update(offsets=equal_offsets(slot * R, R), N=slot * R, mask_slot=slot)
    else:
        kw.update(offsets=ragged_offsets(N, R, w.wid + wid_offset) if ragged else equal_offsets(N, R))
    return w.with_(**kw)
