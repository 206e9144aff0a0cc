"""CPU oracle for paged attention over a blocked KV cache -- TEST INFRASTRUCTURE.

Plain, slow, float64 numpy code that states what the paged path computes.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the library and its Python binding never do, and
this package imports nothing from them.

Every function is pinned by ``tests/test_oracle_*.py`` against facts that do
not come from the oracle itself (format definitions, closed forms, a library
attention routine, brute force at 50 digits, invariants the pages state).
"""
from .reference import (  # noqa: F401
    attend,
    attend_partitioned,
    bf16_to_f64,
    cache_write,
    combine_partials,
    decode_storage,
    dequantize_e4m3,
    dequantize_int8,
    e4m3_to_f64,
    e5m2_to_f64,
    f64_to_e4m3,
    f64_to_e5m2,
    gather_kv,
    new_pool,
    paged_decode,
    paged_varlen,
    quantize_e4m3,
    quantize_int8,
    slot_mapping,
)
