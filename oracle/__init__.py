"""CPU oracle for the paged-KV attention step (float64 numpy).

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``smoke()`` and by the
benchmark's CPU-baseline leg, never by the library or its binding.

Every function is pinned by tests under ``tests/`` against facts the pages
or mathematics fix (brute force on tiny inputs, closed forms, invariances,
the pages' worked arithmetic, library dtype conversions).  No function here
is "parity unpinned".
"""
from .paged_kv import (  # noqa: F401
    F16, BF16, FP8,
    attend, decode_bits, dequant_fp8, gather_scales, gather_sequence, kv_append,
    kv_append_quant, kv_bytes_per_token, lse_merge, paged_attention, partition_partials,
    quantize_e4m3, sequence_kv, tolerance_ok,
)
