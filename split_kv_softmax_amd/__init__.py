"""Python binding of libflare, the gfx950 split-KV / FLARE softmax library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/flare.h``.  PyTorch provides
device memory (outputs and workspace are allocated as torch tensors) and the
stream (``torch.cuda.current_stream()``).  There is no fallback: if the
library is missing or no GPU is present, the calls raise.

Shapes (see the header for the contract):
  encode:     Q [H,M,D] or [B,H,M,D]; K, V [B,H,N,D]  ->  O_part [R,B,H,M,D], L_part [R,B,H,M]
  encode_noalloc: encode with the library's fixed scratch instead of a workspace
  lse_merge:  O_part, L_part                          ->  Z [.., M, D], L [.., M] (+ bf16 Z)
  encode_merge: encode then lse_merge in one call     ->  O_part, L_part, Z, L (+ bf16 Z)
  decode:     Xq [B,H,N,D], Klat [H,M,D] or [B,H,M,D], Z [B,H,M,D] -> Y [B,H,N,D]
  encode_bwd: + Z, L, dZ                              ->  dQ [B,H,M,D], dK, dV [B,H,N,D]
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence, Tuple

import torch  # noqa: F401  (loaded first so the library binds to torch's HIP runtime)

__all__ = ["FlareError", "encode", "encode_noalloc", "lse_merge", "encode_merge", "decode", "encode_bwd", "decode_bwd", "flare_forward",
           "flarepp_forward", "flarepp_backward", "encode_workspace_size", "encode_bwd_workspace_size",
           "decode_bwd_workspace_size", "library_path", "scale_for", "ACCUMULATE_DQ", "ACCUMULATE_DK",
           "ACCUMULATE_DV", "encode_merge", "merge_counters"]

ACCUMULATE_DQ, ACCUMULATE_DK, ACCUMULATE_DV = 1, 2, 4   # flags of encode_bwd (FLARE_BWD_ACCUMULATE_*)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libflare.so")

F32, BF16 = 0, 1
_STATUS = {0: "FLARE_OK", -1: "FLARE_EINVAL", -2: "FLARE_EUNSUPPORTED", -3: "FLARE_EHIP",
           -4: "FLARE_EWORKSPACE"}


class FlareError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -m split_kv_softmax_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    p64 = ctypes.POINTER(ctypes.c_int64)
    lib.flare_encode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, p64, i32]
    lib.flare_encode_workspace_size.restype = sz
    lib.flare_encode.argtypes = [i32, i32, i32, i32, i32, i32, vp, i64, vp, vp, i32, p64, vp, f32, vp, vp,
                                 vp, sz, vp]
    lib.flare_encode.restype = i32
    lib.flare_encode_noalloc.argtypes = [i32, i32, i32, i32, i32, i32, vp, i64, vp, vp, i32, p64, vp, f32, vp, vp,
                                         vp]
    lib.flare_encode_noalloc.restype = i32
    lib.flare_encode_merge.argtypes = [i32, i32, i32, i32, i32, i32, vp, i64, vp, vp, i32, p64, vp, f32, vp,
                                       vp, vp, vp, vp, vp, vp, sz, vp]
    lib.flare_encode_merge.restype = i32
    lib.lse_merge.argtypes = [i32, i64, i32, vp, vp, vp, vp, vp, vp]
    lib.lse_merge.restype = i32
    lib.flare_decode.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, i64, vp, vp, f32, vp, vp]
    lib.flare_decode.restype = i32
    lib.flare_encode_bwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, p64, i32]
    lib.flare_encode_bwd_workspace_size.restype = sz
    lib.flare_encode_bwd.argtypes = [i32, i32, i32, i32, i32, i32, vp, i64, vp, vp, i32, p64, vp, f32, vp,
                                     vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    lib.flare_encode_bwd.restype = i32
    lib.flare_decode_bwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.flare_decode_bwd_workspace_size.restype = sz
    lib.flare_decode_bwd.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, i64, vp, vp, f32, vp, vp, vp, vp, vp,
                                     vp, sz, vp]
    lib.flare_decode_bwd.restype = i32
    lib.flare_last_error.restype = ctypes.c_char_p
    lib.flare_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(st: int):
    if st != 0:
        raise FlareError(st, _load().flare_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _offsets(offsets: Sequence[int]):
    arr = (ctypes.c_int64 * len(offsets))(*[int(o) for o in offsets])
    return arr


def scale_for(D: int) -> float:
    """D^-1/2 rounded to float32 (the pages' scale s)."""
    import numpy as np
    return float(np.float32(1.0) / np.sqrt(np.float32(D)))


_ws_cache: Dict[Tuple[int, int], torch.Tensor] = {}


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    key = (device.index if device.index is not None else torch.cuda.current_device(), 0)
    t = _ws_cache.get(key)
    if t is None or t.numel() < nbytes:
        t = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _ws_cache[key] = t
    return t


def _q_layout(Q: torch.Tensor, B: int, H: int, D: int) -> Tuple[int, int]:
    """(M, batch stride in elements) of a [H,M,D] or [B,H,M,D] query tensor."""
    if Q.dim() == 3:
        if Q.shape[0] != H or Q.shape[2] != D:
            raise ValueError(f"Q shape {tuple(Q.shape)} does not match H={H}, D={D}")
        return Q.shape[1], 0
    if Q.dim() == 4:
        if Q.shape[0] != B or Q.shape[1] != H or Q.shape[3] != D:
            raise ValueError(f"Q shape {tuple(Q.shape)} does not match B={B}, H={H}, D={D}")
        return Q.shape[2], H * Q.shape[2] * D
    raise ValueError("Q must be [H,M,D] or [B,H,M,D]")


def _kv_check(K: torch.Tensor, V: torch.Tensor, Q: torch.Tensor):
    _dev(K, "K")
    _dev(V, "V")
    _dev(Q, "Q")
    if K.dim() != 4 or K.shape != V.shape:
        raise ValueError(f"K {tuple(K.shape)} and V {tuple(V.shape)} must both be [B,H,N,D]")
    if not (K.dtype == V.dtype == Q.dtype):
        raise TypeError("Q, K and V must share one dtype")
    if K.device != Q.device or V.device != Q.device:
        raise ValueError("Q, K and V must be on one device")


def _mask_check(mask: Optional[torch.Tensor], B: int, N: int, device, name="mask"):
    if mask is None:
        return None
    _dev(mask, name)
    if mask.dtype not in (torch.uint8, torch.bool):
        raise TypeError(f"{name} must be uint8 or bool")
    if tuple(mask.shape) != (B, N):
        raise ValueError(f"{name} shape {tuple(mask.shape)} must be ({B}, {N})")
    if mask.device != device:
        raise ValueError(f"{name} must be on the same device")
    return mask.view(torch.uint8) if mask.dtype == torch.bool else mask


def encode_workspace_size(dtype: torch.dtype, B, H, N, M, D, offsets, masked: bool = False) -> int:
    code = BF16 if dtype == torch.bfloat16 else F32
    return int(_load().flare_encode_workspace_size(code, B, H, N, M, D, len(offsets) - 1, _offsets(offsets),
                                                   int(masked)))


def encode(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, offsets: Sequence[int],
           mask: Optional[torch.Tensor] = None, scale: Optional[float] = None,
           O_part: Optional[torch.Tensor] = None, L_part: Optional[torch.Tensor] = None
           ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-partition (O_r, L_r) states of every (batch, head): the local-shard encoder."""
    lib = _load()
    _kv_check(K, V, Q)
    B, H, N, D = K.shape
    M, qbs = _q_layout(Q, B, H, D)
    R = len(offsets) - 1
    mask = _mask_check(mask, B, N, K.device)
    if scale is None:
        scale = scale_for(D)
    dev = K.device
    if O_part is None:
        O_part = torch.empty((R, B, H, M, D), dtype=torch.float32, device=dev)
    if L_part is None:
        L_part = torch.empty((R, B, H, M), dtype=torch.float32, device=dev)
    if tuple(O_part.shape) != (R, B, H, M, D) or tuple(L_part.shape) != (R, B, H, M):
        raise ValueError("O_part / L_part have the wrong shape")
    if O_part.dtype != torch.float32 or L_part.dtype != torch.float32:
        raise TypeError("O_part / L_part must be float32")
    _dev(O_part, "O_part")
    _dev(L_part, "L_part")
    offs = _offsets(offsets)
    code = _dtype_code(K)
    nbytes = int(lib.flare_encode_workspace_size(code, B, H, N, M, D, R, offs, int(mask is not None)))
    ws = _workspace(nbytes, dev)
    with torch.cuda.device(dev):
        _check(lib.flare_encode(code, B, H, N, M, D, _ptr(Q), qbs, _ptr(K), _ptr(V), R, offs, _ptr(mask),
                                float(scale), _ptr(O_part), _ptr(L_part), _ptr(ws), nbytes, _stream()))
    return O_part, L_part


NOALLOC_SCRATCH_BYTES = 16 << 20    # FLARE_NOALLOC_SCRATCH_BYTES


def encode_noalloc(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, offsets: Sequence[int],
                   mask: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                   O_part: Optional[torch.Tensor] = None, L_part: Optional[torch.Tensor] = None
                   ) -> Tuple[torch.Tensor, torch.Tensor]:
    """encode through flare_encode_noalloc: the library's fixed per-device scratch in place of a
    workspace (for callers that cannot allocate; pass O_part and L_part to allocate nothing here)."""
    lib = _load()
    _kv_check(K, V, Q)
    B, H, N, D = K.shape
    M, qbs = _q_layout(Q, B, H, D)
    R = len(offsets) - 1
    mask = _mask_check(mask, B, N, K.device)
    if scale is None:
        scale = scale_for(D)
    dev = K.device
    if O_part is None:
        O_part = torch.empty((R, B, H, M, D), dtype=torch.float32, device=dev)
    if L_part is None:
        L_part = torch.empty((R, B, H, M), dtype=torch.float32, device=dev)
    if tuple(O_part.shape) != (R, B, H, M, D) or tuple(L_part.shape) != (R, B, H, M):
        raise ValueError("O_part / L_part have the wrong shape")
    if O_part.dtype != torch.float32 or L_part.dtype != torch.float32:
        raise TypeError("O_part / L_part must be float32")
    _dev(O_part, "O_part")
    _dev(L_part, "L_part")
    with torch.cuda.device(dev):
        _check(lib.flare_encode_noalloc(_dtype_code(K), B, H, N, M, D, _ptr(Q), qbs, _ptr(K), _ptr(V), R,
                                        _offsets(offsets), _ptr(mask), float(scale), _ptr(O_part), _ptr(L_part),
                                        _stream()))
    return O_part, L_part


_cnt_cache: Dict[int, torch.Tensor] = {}


def merge_counters(n: int, device) -> torch.Tensor:
    """The per-device array of arrival counters encode_merge hands to the library
    (zeroed once when allocated; every call leaves it zero)."""
    key = device.index if device.index is not None else torch.cuda.current_device()
    t = _cnt_cache.get(key)
    if t is None or t.numel() < n:
        t = torch.zeros(max(n, 1024), dtype=torch.int32, device=device)
        _cnt_cache[key] = t
    return t


def encode_merge(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, offsets: Sequence[int],
                 mask: Optional[torch.Tensor] = None, scale: Optional[float] = None, want_bf16: bool = False,
                 O_part: Optional[torch.Tensor] = None, L_part: Optional[torch.Tensor] = None,
                 Z: Optional[torch.Tensor] = None, L: Optional[torch.Tensor] = None,
                 Z_bf16: Optional[torch.Tensor] = None, counters: Optional[torch.Tensor] = None):
    """encode then lse_merge in one C-ABI call (one launch on the matrix-core path):
    -> (O_part, L_part, Z, L, Z_bf16 or None).  counters: int32 [>= B*H*(R+1)] zeros
    (default: a per-device array kept by this module)."""
    lib = _load()
    _kv_check(K, V, Q)
    B, H, N, D = K.shape
    M, qbs = _q_layout(Q, B, H, D)
    R = len(offsets) - 1
    mask = _mask_check(mask, B, N, K.device)
    if scale is None:
        scale = scale_for(D)
    dev = K.device
    if O_part is None:
        O_part = torch.empty((R, B, H, M, D), dtype=torch.float32, device=dev)
    if L_part is None:
        L_part = torch.empty((R, B, H, M), dtype=torch.float32, device=dev)
    if Z is None:
        Z = torch.empty((B, H, M, D), dtype=torch.float32, device=dev)
    if L is None:
        L = torch.empty((B, H, M), dtype=torch.float32, device=dev)
    if want_bf16 and Z_bf16 is None:
        Z_bf16 = torch.empty((B, H, M, D), dtype=torch.bfloat16, device=dev)
    if tuple(O_part.shape) != (R, B, H, M, D) or tuple(L_part.shape) != (R, B, H, M):
        raise ValueError("O_part / L_part have the wrong shape")
    if tuple(Z.shape) != (B, H, M, D) or tuple(L.shape) != (B, H, M):
        raise ValueError("Z / L have the wrong shape")
    if Z_bf16 is not None and (tuple(Z_bf16.shape) != (B, H, M, D) or Z_bf16.dtype != torch.bfloat16):
        raise ValueError("Z_bf16 must be bfloat16 [B,H,M,D]")
    for t, name in ((O_part, "O_part"), (L_part, "L_part"), (Z, "Z"), (L, "L")):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
        _dev(t, name)
    ncnt = B * H * (R + 1)
    if counters is None:
        counters = merge_counters(ncnt, dev)
    if counters.dtype != torch.int32 or counters.numel() < ncnt:
        raise ValueError("counters must be int32 with at least B*H*(R+1) entries")
    _dev(counters, "counters")
    offs = _offsets(offsets)
    code = _dtype_code(K)
    nbytes = int(lib.flare_encode_workspace_size(code, B, H, N, M, D, R, offs, int(mask is not None)))
    ws = _workspace(nbytes, dev)
    with torch.cuda.device(dev):
        _check(lib.flare_encode_merge(code, B, H, N, M, D, _ptr(Q), qbs, _ptr(K), _ptr(V), R, offs, _ptr(mask),
                                      float(scale), _ptr(O_part), _ptr(L_part), _ptr(Z), _ptr(L), _ptr(Z_bf16),
                                      _ptr(counters), _ptr(ws), nbytes, _stream()))
    return O_part, L_part, Z, L, Z_bf16


def lse_merge(O_part: torch.Tensor, L_part: torch.Tensor, want_bf16: bool = False,
              Z: Optional[torch.Tensor] = None, L: Optional[torch.Tensor] = None,
              Z_bf16: Optional[torch.Tensor] = None):
    """Tree merge of R partition states -> (Z, L, Z_bf16 or None)."""
    lib = _load()
    _dev(O_part, "O_part")
    _dev(L_part, "L_part")
    if O_part.dtype != torch.float32 or L_part.dtype != torch.float32:
        raise TypeError("O_part / L_part must be float32")
    if O_part.dim() < 2 or tuple(O_part.shape[:-1]) != tuple(L_part.shape):
        raise ValueError(f"O_part {tuple(O_part.shape)} and L_part {tuple(L_part.shape)} disagree")
    R = O_part.shape[0]
    D = O_part.shape[-1]
    rows = L_part[0].numel()
    dev = O_part.device
    if Z is None:
        Z = torch.empty(O_part.shape[1:], dtype=torch.float32, device=dev)
    if L is None:
        L = torch.empty(L_part.shape[1:], dtype=torch.float32, device=dev)
    if tuple(Z.shape) != tuple(O_part.shape[1:]) or tuple(L.shape) != tuple(L_part.shape[1:]):
        raise ValueError("Z / L have the wrong shape")
    if want_bf16 and Z_bf16 is None:
        Z_bf16 = torch.empty(O_part.shape[1:], dtype=torch.bfloat16, device=dev)
    if Z_bf16 is not None and tuple(Z_bf16.shape) != tuple(Z.shape):
        raise ValueError("Z_bf16 has the wrong shape")
    with torch.cuda.device(dev):
        _check(lib.lse_merge(R, rows, D, _ptr(O_part), _ptr(L_part), _ptr(Z), _ptr(L), _ptr(Z_bf16),
                             _stream()))
    return Z, L, Z_bf16


def decode(Xq: torch.Tensor, Klat: torch.Tensor, Z: torch.Tensor, scale: Optional[float] = None,
           token_mask: Optional[torch.Tensor] = None, Y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = softmax_m(scale Xq Klat^T) Z for every token."""
    lib = _load()
    _dev(Xq, "Xq")
    _dev(Klat, "Klat")
    _dev(Z, "Z")
    if Xq.dim() != 4:
        raise ValueError("Xq must be [B,H,N,D]")
    B, H, N, D = Xq.shape
    if Klat.dtype != Xq.dtype:
        raise TypeError("Xq and Klat must share one dtype")
    M, kbs = _q_layout(Klat, B, H, D)
    if tuple(Z.shape) != (B, H, M, D) or Z.dtype != torch.float32:
        raise ValueError(f"Z must be float32 [B,H,M,D] = ({B},{H},{M},{D})")
    token_mask = _mask_check(token_mask, B, N, Xq.device, "token_mask")
    if scale is None:
        scale = scale_for(D)
    if Y is None:
        Y = torch.empty_like(Xq)
    if tuple(Y.shape) != tuple(Xq.shape) or Y.dtype != Xq.dtype:
        raise ValueError("Y has the wrong shape or dtype")
    _dev(Y, "Y")
    with torch.cuda.device(Xq.device):
        _check(lib.flare_decode(_dtype_code(Xq), B, H, N, M, D, _ptr(Xq), _ptr(Klat), kbs, _ptr(Z),
                                _ptr(token_mask), float(scale), _ptr(Y), _stream()))
    return Y


def encode_bwd_workspace_size(dtype: torch.dtype, B, H, N, M, D, offsets, masked: bool = False) -> int:
    code = BF16 if dtype == torch.bfloat16 else F32
    return int(_load().flare_encode_bwd_workspace_size(code, B, H, N, M, D, len(offsets) - 1,
                                                       _offsets(offsets), int(masked)))


def encode_bwd(Q, K, V, offsets, mask, scale, Z, L, dZ, dQ=None, dK=None, dV=None, dQ_cast=None,
               flags: int = 0):
    """Encoder gradients with the global statistics -> (dQ [B,H,M,D] f32, dK, dV).

    ``flags`` (ACCUMULATE_DQ / ACCUMULATE_DK / ACCUMULATE_DV) add into the given dQ / dK / dV
    instead of overwriting them; ``dQ_cast`` (a [B,H,M,D] tensor in the input dtype) also
    receives dQ.
    """
    lib = _load()
    _kv_check(K, V, Q)
    B, H, N, D = K.shape
    M, qbs = _q_layout(Q, B, H, D)
    R = len(offsets) - 1
    mask = _mask_check(mask, B, N, K.device)
    for t, nm in ((Z, "Z"), (L, "L"), (dZ, "dZ")):
        _dev(t, nm)
    if tuple(Z.shape) != (B, H, M, D) or Z.dtype != torch.float32:
        raise ValueError("Z must be float32 [B,H,M,D]")
    if tuple(L.shape) != (B, H, M) or L.dtype != torch.float32:
        raise ValueError("L must be float32 [B,H,M]")
    if tuple(dZ.shape) != (B, H, M, D) or dZ.dtype != K.dtype:
        raise ValueError("dZ must be [B,H,M,D] in the input dtype")
    if scale is None:
        scale = scale_for(D)
    dev = K.device
    dQ = torch.empty((B, H, M, D), dtype=torch.float32, device=dev) if dQ is None else dQ
    dK = torch.empty_like(K) if dK is None else dK
    dV = torch.empty_like(V) if dV is None else dV
    if tuple(dQ.shape) != (B, H, M, D) or dQ.dtype != torch.float32:
        raise ValueError("dQ must be float32 [B,H,M,D]")
    if dK.shape != K.shape or dV.shape != V.shape or dK.dtype != K.dtype or dV.dtype != K.dtype:
        raise ValueError("dK / dV must match K / V")
    if dQ_cast is not None:
        _dev(dQ_cast, "dQ_cast")
        if tuple(dQ_cast.shape) != (B, H, M, D) or dQ_cast.dtype != K.dtype:
            raise ValueError("dQ_cast must be [B,H,M,D] in the input dtype")
    offs = _offsets(offsets)
    code = _dtype_code(K)
    nbytes = int(lib.flare_encode_bwd_workspace_size(code, B, H, N, M, D, R, offs, int(mask is not None)))
    ws = _workspace(nbytes, dev)
    with torch.cuda.device(dev):
        _check(lib.flare_encode_bwd(code, B, H, N, M, D, _ptr(Q), qbs, _ptr(K), _ptr(V), R, offs, _ptr(mask),
                                    float(scale), _ptr(Z), _ptr(L), _ptr(dZ), _ptr(dQ), _ptr(dK), _ptr(dV),
                                    _ptr(dQ_cast), int(flags), _ptr(ws), nbytes, _stream()))
    return dQ, dK, dV


def decode_bwd_workspace_size(dtype: torch.dtype, B, H, N, M, D, masked: bool = False) -> int:
    code = BF16 if dtype == torch.bfloat16 else F32
    return int(_load().flare_decode_bwd_workspace_size(code, B, H, N, M, D, int(masked)))


def decode_bwd(Xq, Klat, Z, scale, dY, token_mask=None, dXq=None, dKlat=None, dZ=None, dZ_cast=None):
    """Decode gradients -> (dXq [B,H,N,D] in the input dtype, dKlat [B,H,M,D] f32, dZ [B,H,M,D] f32)."""
    lib = _load()
    for t, nm in ((Xq, "Xq"), (Klat, "Klat"), (Z, "Z"), (dY, "dY")):
        _dev(t, nm)
    if Xq.dim() != 4:
        raise ValueError("Xq must be [B,H,N,D]")
    B, H, N, D = Xq.shape
    if Klat.dtype != Xq.dtype or dY.dtype != Xq.dtype:
        raise TypeError("Xq, Klat and dY must share one dtype")
    if dY.shape != Xq.shape:
        raise ValueError("dY must match Xq")
    M, kbs = _q_layout(Klat, B, H, D)
    if tuple(Z.shape) != (B, H, M, D) or Z.dtype != torch.float32:
        raise ValueError(f"Z must be float32 [B,H,M,D] = ({B},{H},{M},{D})")
    token_mask = _mask_check(token_mask, B, N, Xq.device, "token_mask")
    if scale is None:
        scale = scale_for(D)
    dev = Xq.device
    dXq = torch.empty_like(Xq) if dXq is None else dXq
    dKlat = torch.empty((B, H, M, D), dtype=torch.float32, device=dev) if dKlat is None else dKlat
    dZ = torch.empty((B, H, M, D), dtype=torch.float32, device=dev) if dZ is None else dZ
    if dXq.shape != Xq.shape or dXq.dtype != Xq.dtype:
        raise ValueError("dXq must match Xq")
    for t, nm in ((dKlat, "dKlat"), (dZ, "dZ")):
        _dev(t, nm)
        if tuple(t.shape) != (B, H, M, D) or t.dtype != torch.float32:
            raise ValueError(f"{nm} must be float32 [B,H,M,D]")
    if dZ_cast is not None:
        _dev(dZ_cast, "dZ_cast")
        if tuple(dZ_cast.shape) != (B, H, M, D) or dZ_cast.dtype != Xq.dtype:
            raise ValueError("dZ_cast must be [B,H,M,D] in the input dtype")
    code = _dtype_code(Xq)
    nbytes = int(lib.flare_decode_bwd_workspace_size(code, B, H, N, M, D, int(token_mask is not None)))
    ws = _workspace(nbytes, dev)
    with torch.cuda.device(dev):
        _check(lib.flare_decode_bwd(code, B, H, N, M, D, _ptr(Xq), _ptr(Klat), kbs, _ptr(Z), _ptr(token_mask),
                                    float(scale), _ptr(dY), _ptr(dXq), _ptr(dKlat), _ptr(dZ), _ptr(dZ_cast),
                                    _ptr(ws), nbytes, _stream()))
    return dXq, dKlat, dZ


def flare_forward(Q, K, V, offsets, mask=None, scale=None, token_mask=None, fused=False):
    """FLARE block mixer: Z = merge(encode(Q, K, V)); Y = decode(K, Q, Z).
    fused=True makes the encode and the merge one call, flare_encode_merge (same
    results; one launch, but slower than two on MI355X at the measured shapes)."""
    if fused:
        O_part, L_part, Z, L, _ = encode_merge(Q, K, V, offsets, mask, scale)
    else:
        O_part, L_part = encode(Q, K, V, offsets, mask, scale)
        Z, L, _ = lse_merge(O_part, L_part)
    Y = decode(K, Q, Z, scale, token_mask)
    return {"O_part": O_part, "L_part": L_part, "Z": Z, "L": L, "Y": Y}


def flarepp_backward(fwd, Qt, Kt, Vt, K, V, offsets, dY, scale=None):
    """Gradients of sum(dY * Y) for the FLARE++ chain, from the saved forward ``fwd``
    (the dict flarepp_forward returns): three C-ABI calls.

    decoder backward at (K, Q(X), Z) -> dK, dQ(X) (decoder part), dZ (also in the
    input dtype); physical-value encoder backward with its own (Z, L), adding into
    dQ(X) and dK and writing dV, and writing dQ(X) in the input dtype; query-synthesis
    encoder backward with its own (Q(X), L) and that dQ(X) -> dQt, dKt, dVt.
    Q(X) enters the second encoder and the decoder rounded to the input dtype; its
    gradient passes the rounding unchanged.

    Shared projections (Kt is K and Vt is V): the query-synthesis encoder's key and
    value gradients add into dK and dV, and dKt, dVt are those same tensors.
    """
    QXin = fwd["QX_in"]
    shared = Kt is K and Vt is V
    dZc = torch.empty_like(fwd["Z"], dtype=K.dtype)
    dK, dQX, _ = decode_bwd(K, QXin, fwd["Z"], scale, dY, dZ_cast=dZc)
    dQXc = torch.empty_like(dQX, dtype=K.dtype)
    _, dK, dV = encode_bwd(QXin, K, V, offsets, None, scale, fwd["Z"], fwd["L"], dZc, dQ=dQX, dK=dK,
                           dQ_cast=dQXc, flags=ACCUMULATE_DQ | ACCUMULATE_DK)
    if shared:
        dQt, dKt, dVt = encode_bwd(Qt, K, V, offsets, None, scale, fwd["QX"], fwd["QX_L"], dQXc, dK=dK, dV=dV,
                                   flags=ACCUMULATE_DK | ACCUMULATE_DV)
    else:
        dQt, dKt, dVt = encode_bwd(Qt, Kt, Vt, offsets, None, scale, fwd["QX"], fwd["QX_L"], dQXc)
    return {"dQt": dQt, "dKt": dKt, "dVt": dVt, "dK": dK, "dV": dV, "dQX": dQX}


def flarepp_forward(Qt, Kt, Vt, K, V, offsets, scale=None, fused=False):
    """FLARE++: Q(X) = merge(encode(Qt, Kt, Vt)); Z = merge(encode(Q(X), K, V)); Y = decode(K, Q(X), Z).

    The dynamic queries are consumed in the input dtype (the merge writes a
    bfloat16 copy next to the float32 result for bfloat16 inputs).  fused=True
    makes each encode and its merge one call, flare_encode_merge (same results).
    The shared-projection variant passes K and V as Kt and Vt.
    """
    bf16 = K.dtype == torch.bfloat16
    if fused:
        O1, L1, QX, QX_L, QXb = encode_merge(Qt, Kt, Vt, offsets, None, scale, want_bf16=bf16)
    else:
        O1, L1 = encode(Qt, Kt, Vt, offsets, None, scale)
        QX, QX_L, QXb = lse_merge(O1, L1, want_bf16=bf16)
    QXin = QXb if QXb is not None else QX
    if fused:
        O2, L2, Z, L, _ = encode_merge(QXin, K, V, offsets, None, scale)
    else:
        O2, L2 = encode(QXin, K, V, offsets, None, scale)
        Z, L, _ = lse_merge(O2, L2)
    Y = decode(K, QXin, Z, scale)
    return {"QX": QX, "QX_L": QX_L, "QX_in": QXin, "QX_O_part": O1, "QX_L_part": L1,
            "O_part": O2, "L_part": L2, "Z": Z, "L": L, "Y": Y}
