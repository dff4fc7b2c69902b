"""CPU oracle (float64 numpy) and decimal brute force for the split-KV softmax path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its binding.
"""
from . import flare_ref  # noqa: F401
