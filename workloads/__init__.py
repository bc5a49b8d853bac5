"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the bench.

Random draws and data layout only; no attention arithmetic lives here.
"""
from . import gen, cases  # noqa: F401
from .cases import (PrefillCase, DecodeCase, make_prefill, make_decode, prefill_tiny,  # noqa: F401
                    prefill_llama8b, prefill_extreme, decode_llama8b, decode_ragged)
