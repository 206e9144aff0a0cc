"""libpagedattn: PagedAttention over a blocked KV cache on MI355X (gfx950).

The computation lives in the HIP kernels of ``libpagedattn.so`` (built from
``csrc/`` by ``python -m paged_kv_cache_251_amd.build``); this package is its
ctypes binding.
"""
from .binding import (  # noqa: F401
    LIB_PATH,
    PA_BF16,
    PA_F32,
    PA_FP8_E4M3,
    PA_FP8_E5M2,
    PA_INT8,
    BlockManager,
    PagedAttnError,
    Scheduler,
    abi_version,
    alloc_workspace,
    auto_partition,
    copy_blocks,
    int8_scale_order,
    kv_cache_write,
    lib,
    new_scaled_pools,
    paged_attention_decode,
    paged_attention_decode_append,
    paged_attention_decode_static,
    paged_attention_varlen,
    scaled_pool_split,
    slot_mapping,
    workspace_size,
)
