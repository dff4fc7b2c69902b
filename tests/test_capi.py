"""Host-side checks of the C ABI (CPU only): the library loads, exports every
declared entry point, and validates arguments before touching the GPU.

The validation paths return before any HIP call, so they run without a GPU;
device pointers passed here are placeholders that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "flare.h")
LIB = os.path.join(ROOT, "split_kv_softmax_amd", "libflare.so")

EINVAL, EUNSUP, EWS = -1, -2, -4
FAKE = ctypes.c_void_p(0x7f0000000000)   # aligned placeholder, never dereferenced


def declared_functions():
    txt = open(HDR).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b((?:flare|lse)_\w+)\s*\(", txt, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libflare.so is not built (run python -m split_kv_softmax_amd.build)")
    L = ctypes.CDLL(LIB)
    p64 = ctypes.POINTER(ctypes.c_int64)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.flare_encode.argtypes = [i32, i32, i32, i32, i32, i32, vp, i64, vp, vp, i32, p64, vp, f32, vp, vp, vp, sz, vp]
    L.flare_encode_noalloc.argtypes = [i32, i32, i32, i32, i32, i32, vp, i64, vp, vp, i32, p64, vp, f32, vp, vp, vp]
    L.flare_encode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, p64, i32]
    L.flare_encode_workspace_size.restype = sz
    L.lse_merge.argtypes = [i32, i64, i32, vp, vp, vp, vp, vp, vp]
    L.flare_encode_merge.argtypes = [i32, i32, i32, i32, i32, i32, vp, i64, vp, vp, i32, p64, vp, f32, vp, vp, vp,
                                     vp, vp, vp, vp, sz, vp]
    L.flare_decode.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, i64, vp, vp, f32, vp, vp]
    L.flare_encode_bwd.argtypes = [i32, i32, i32, i32, i32, i32, vp, i64, vp, vp, i32, p64, vp, f32, vp, vp, vp,
                                   vp, vp, vp, vp, i32, vp, sz, vp]
    L.flare_decode_bwd.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, i64, vp, vp, f32, vp, vp, vp, vp, vp,
                                   vp, sz, vp]
    L.flare_decode_bwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.flare_decode_bwd_workspace_size.restype = sz
    L.flare_encode_bwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, p64, i32]
    L.flare_encode_bwd_workspace_size.restype = sz
    L.flare_last_error.restype = ctypes.c_char_p
    L.flare_version.restype = ctypes.c_char_p
    return L


def offs(*v):
    return (ctypes.c_int64 * len(v))(*v)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"flare_encode", "flare_encode_merge", "lse_merge", "flare_decode", "flare_encode_bwd"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert b"gfx950" in lib.flare_version()


def _enc(lib, o, N=1024, M=64, D=64, dt=1, ws=None, nbytes=0, Q=FAKE):
    return lib.flare_encode(dt, 1, 1, N, M, D, Q, 0, FAKE, FAKE, len(o) - 1, o, None, 0.125, FAKE, FAKE, ws, nbytes,
                            None)


def test_offsets_are_validated(lib):
    assert _enc(lib, offs(1, 500, 1024)) == EINVAL                  # must start at 0
    assert b"offsets[0]" in lib.flare_last_error()
    assert _enc(lib, offs(0, 600, 500, 1024)) == EINVAL             # overlapping / unsorted
    assert b"disjoint" in lib.flare_last_error()
    assert _enc(lib, offs(0, 500, 1000)) == EINVAL                  # does not end at N
    assert lib.flare_encode(1, 1, 1, 1024, 64, 64, FAKE, 0, FAKE, FAKE, 0, offs(0), None, 0.1, FAKE, FAKE, None, 0,
                            None) == EINVAL                           # R = 0


def test_shapes_pointers_and_scale_are_validated(lib):
    assert _enc(lib, offs(0, 1024), D=6) == EUNSUP
    assert _enc(lib, offs(0, 1024), D=512) == EUNSUP
    assert _enc(lib, offs(0, 1024), dt=7) == EINVAL
    assert _enc(lib, offs(0, 1024), Q=None) == EINVAL
    assert lib.flare_encode(1, 1, 1, 1024, 64, 64, FAKE, 0, FAKE, FAKE, 1, offs(0, 1024), None, float("nan"), FAKE,
                            FAKE, None, 0, None) == EINVAL
    mis = ctypes.c_void_p(0x7f0000000002)
    assert lib.flare_encode(1, 1, 1, 1024, 64, 64, mis, 0, FAKE, FAKE, 1, offs(0, 1024), None, 0.1, FAKE, FAKE,
                            None, 0, None) == EINVAL                  # misaligned for the matrix-core path
    assert lib.lse_merge(0, 10, 64, FAKE, FAKE, FAKE, FAKE, None, None) == EINVAL
    assert lib.lse_merge(4, 10, 6, FAKE, FAKE, FAKE, FAKE, None, None) == EUNSUP
    assert lib.flare_decode(1, 1, 1, 100, 300, 64, FAKE, FAKE, 0, FAKE, None, 0.1, FAKE, None) == EUNSUP
    assert lib.flare_decode(1, 1, 1, 100, 64, 64, None, FAKE, 0, FAKE, None, 0.1, FAKE, None) == EINVAL


def test_workspace_contract(lib):
    o = offs(0, 40000, 80000)
    n = lib.flare_encode_workspace_size(1, 1, 2, 80000, 128, 64, 2, o, 0)
    assert n > 0                                       # long partitions are split into chunks
    assert n == lib.flare_encode_workspace_size(1, 1, 2, 80000, 128, 64, 2, o, 0)
    assert lib.flare_encode_workspace_size(1, 1, 2, 80000, 128, 64, 2, o, 1) > n     # room for mask words
    assert lib.flare_encode(1, 1, 2, 80000, 128, 64, FAKE, 0, FAKE, FAKE, 2, o, None, 0.125, FAKE, FAKE, None, 0,
                            None) == EWS
    assert b"workspace" in lib.flare_last_error()
    assert lib.flare_encode(1, 1, 2, 80000, 128, 64, FAKE, 0, FAKE, FAKE, 2, o, None, 0.125, FAKE, FAKE, FAKE, n - 1,
                            None) == EWS
    # a small problem needs none, and invalid arguments report 0
    assert lib.flare_encode_workspace_size(1, 1, 1, 1024, 64, 64, 1, offs(0, 1024), 0) == 0
    assert lib.flare_encode_workspace_size(1, 1, 1, 1024, 64, 64, 2, offs(0, 900, 800), 0) == 0


def test_backward_validates_offsets(lib):
    assert lib.flare_encode_bwd(1, 1, 1, 100, 64, 64, FAKE, 0, FAKE, FAKE, 2, offs(0, 70, 60), None, 0.1, FAKE, FAKE,
                                FAKE, FAKE, FAKE, FAKE, None, 0, None, 0, None) == EINVAL
    # unknown flags are rejected before anything else runs
    assert lib.flare_encode_bwd(1, 1, 1, 100, 64, 64, FAKE, 0, FAKE, FAKE, 2, offs(0, 50, 100), None, 0.1, FAKE,
                                FAKE, FAKE, FAKE, FAKE, FAKE, None, 8, None, 0, None) == EINVAL
    assert b"flags" in lib.flare_last_error()
    # the three accumulate flags pass that check (and stop at the missing workspace)
    assert lib.flare_encode_bwd(1, 1, 1, 100, 64, 64, FAKE, 0, FAKE, FAKE, 2, offs(0, 50, 100), None, 0.1, FAKE,
                                FAKE, FAKE, FAKE, FAKE, FAKE, None, 7, None, 0, None) == EWS


def test_decode_backward_validates(lib):
    """Shape, pointer and workspace checks of the decode backward, before any launch."""
    assert lib.flare_decode_bwd(1, 1, 1, 100, 300, 64, FAKE, FAKE, 0, FAKE, None, 0.1, FAKE, FAKE, FAKE, FAKE,
                                None, FAKE, 1 << 20, None) == EUNSUP
    assert lib.flare_decode_bwd(1, 1, 1, 100, 64, 64, FAKE, None, 0, FAKE, None, 0.1, FAKE, FAKE, FAKE, FAKE,
                                None, FAKE, 1 << 20, None) == EINVAL
    n = lib.flare_decode_bwd_workspace_size(1, 1, 2, 1000, 64, 64, 0)
    assert n > 0 and n == lib.flare_decode_bwd_workspace_size(1, 1, 2, 1000, 64, 64, 0)
    assert lib.flare_decode_bwd(1, 1, 2, 1000, 64, 64, FAKE, FAKE, 0, FAKE, None, 0.1, FAKE, FAKE, FAKE, FAKE,
                                None, FAKE, n - 1, None) == EWS
    assert lib.flare_decode_bwd_workspace_size(1, 1, 2, 1000, 300, 64, 0) == 0     # invalid shape -> 0


def _encm(lib, o, Z=FAKE, L=FAKE, Zb=None, cnt=FAKE, N=1024, ws=None, nbytes=0):
    return lib.flare_encode_merge(1, 1, 1, N, 64, 64, FAKE, 0, FAKE, FAKE, len(o) - 1, o, None, 0.125, FAKE, FAKE,
                                  Z, L, Zb, cnt, ws, nbytes, None)


def test_encode_merge_validates(lib):
    """The merged call checks what flare_encode checks, plus its merge outputs and counters."""
    assert _encm(lib, offs(0, 600, 500, 1024)) == EINVAL            # offsets as flare_encode
    assert b"disjoint" in lib.flare_last_error()
    assert _encm(lib, offs(0, 1024), Z=None) == EINVAL
    assert _encm(lib, offs(0, 1024), L=None) == EINVAL
    assert _encm(lib, offs(0, 1024), cnt=None) == EINVAL
    assert b"counters" in lib.flare_last_error()
    assert _encm(lib, offs(0, 1024), Z=ctypes.c_void_p(0x7f0000000008)) == EINVAL      # Z 16-byte aligned
    assert _encm(lib, offs(0, 1024), Zb=ctypes.c_void_p(0x7f0000000004)) == EINVAL     # Z_bf16 8-byte aligned
    assert _encm(lib, offs(0, 1024), cnt=ctypes.c_void_p(0x7f0000000002)) == EINVAL    # counters 4-byte aligned
    o = offs(0, 40000, 80000)
    n = lib.flare_encode_workspace_size(1, 1, 1, 80000, 64, 64, 2, o, 0)
    assert n > 0 and _encm(lib, o, N=80000, ws=FAKE, nbytes=n - 1) == EWS               # same workspace as encode


def test_noalloc_encoder_rejects_workspace_beyond_its_scratch(lib):
    """flare_encode_noalloc refuses (before any launch or HIP call) arguments whose workspace
    exceeds its fixed scratch: one (batch, head) slice of 2^20 tokens, 256 latent rows at head
    dim 128, split into 256 chunks whose partial states need 32 MiB; invalid arguments get
    flare_encode's own status."""
    N = 1 << 20
    o = offs(0, N)
    need = lib.flare_encode_workspace_size(1, 1, 1, N, 256, 128, 1, o, 0)
    assert need > 16 << 20
    st = lib.flare_encode_noalloc(1, 1, 1, N, 256, 128, FAKE, 0, FAKE, FAKE, 1, o, None, 0.088, FAKE, FAKE, None)
    assert st == EWS
    assert b"flare_encode_noalloc" in lib.flare_last_error() and b"scratch" in lib.flare_last_error()
    st = lib.flare_encode_noalloc(1, 1, 1, 1024, 64, 64, FAKE, 0, FAKE, FAKE, 2, offs(0, 600, 500), None, 0.125,
                                  FAKE, FAKE, None)
    assert st == EINVAL and b"offsets" in lib.flare_last_error()
