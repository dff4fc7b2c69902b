"""The oracle and the HIP path share no code, and the product never reaches the oracle."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sources(d, exts):
    for dp, _, fs in os.walk(os.path.join(ROOT, d)):
        for f in fs:
            if f.endswith(exts):
                yield os.path.join(dp, f)


def test_oracle_imports_nothing_from_the_library():
    for p in _sources("oracle", (".py", ".c", ".h")):
        txt = open(p).read()
        assert "split_kv_softmax_amd" not in txt, p
        assert not re.search(r"^\s*(from|import)\s+workloads", txt, re.M), p


def test_library_never_reaches_the_oracle():
    for p in _sources("split_kv_softmax_amd", (".py", ".hip", ".cpp", ".h")):
        txt = open(p).read()
        assert not re.search(r"^\s*(from|import)\s+oracle", txt, re.M), p
        assert "oracle/" not in txt and "flare_ref" not in txt, p
    for p in _sources("workloads", (".py",)):
        txt = open(p).read()
        assert not re.search(r"^\s*(from|import)\s+(oracle|split_kv_softmax_amd)", txt, re.M), p


def test_binding_fails_loudly_without_the_library():
    """No fallback: a missing libflare raises ImportError, and host tensors are refused."""
    import pytest
    import torch

    import split_kv_softmax_amd as fl
    saved = (fl._LIB_PATH, fl._lib)
    try:
        fl._LIB_PATH = os.path.join(ROOT, "split_kv_softmax_amd", "no_such_libflare.so")
        fl._lib = None
        with pytest.raises(ImportError):
            fl._load()
    finally:
        fl._LIB_PATH, fl._lib = saved
    if os.path.exists(fl.library_path()):
        Q = torch.zeros((2, 64, 64), dtype=torch.bfloat16)
        K = torch.zeros((1, 2, 128, 64), dtype=torch.bfloat16)
        with pytest.raises(ValueError, match="GPU tensor"):
            fl.encode(Q, K, K, [0, 128])
        with pytest.raises(ValueError, match="GPU tensor"):
            fl.encode_merge(Q, K, K, [0, 128])
