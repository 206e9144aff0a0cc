"""Seeded synthetic inputs shared by the oracle-side tests and the HIP path.

Nothing here computes any part of paged attention: the module draws sequence
lengths, physical block assignments and q/K/V values in their storage dtype,
and describes which token rows a cache write carries.  Slot arithmetic, the
fp8 cast, the gather and the attention itself live on the two sides that are
compared (``oracle/`` on the CPU, ``libpagedattn`` on the GPU).
"""
from .generate import (  # noqa: F401
    CONFIG_NAMES,
    POISON_BITS,
    STORAGE,
    Workload,
    WritePlan,
    make_config,
    make_workload,
    queries,
    seq_kv,
    write_plan,
)
