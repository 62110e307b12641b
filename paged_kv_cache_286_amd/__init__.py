"""Paged-KV attention step for MI355X (gfx950).

The compute path is the C-ABI library ``libpagedkv.so`` (hand-written HIP);
``paged_kv_cache_286_amd.pagedkv`` is its thin ctypes binding and raises on
import when the library has not been built.  ``workloads`` draws seeded
synthetic steps; ``blocks`` is the host-side block manager.
"""
