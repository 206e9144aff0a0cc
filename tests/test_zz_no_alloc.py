"""The decode entry point that allocates nothing (needs an MI355X).

paged_attention_decode_static keeps its split-KV partials in the library's own per-GPU scratch
array instead of a caller workspace.  Through the C ABI it must give exactly what
paged_attention_decode gives with a caller workspace and the same partition size, on two calls in
a row (the second smaller, so it runs over what the first left in the array), including a split
whose partials fill most of the array; a split that needs more than the array holds is refused on
the host.
"""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_251_amd as pa
from gpu_harness import DEV, DeviceBatch
from workloads import make_workload

pytestmark = pytest.mark.gpu

LIMIT = 32 << 20  # PA_STATIC_WORKSPACE_BYTES


def _static(b, partition, out, max_context_len=None):
    w = b.w
    mcl = w.max_context_len if max_context_len is None else max_context_len
    lib = pa.lib()
    n, hq, d = b.q.shape
    st = lib.paged_attention_decode_static(
        out.data_ptr(), b.q.data_ptr(), b.pk.data_ptr(), b.pv.data_ptr(), b.tables.data_ptr(), b.tables.shape[1],
        b.lens.data_ptr(), n, w.num_kv_heads, w.gqa_group, d, w.block_size, w.num_blocks, mcl,
        ctypes.c_float(w.scale), pa.binding.dtype_code(b.q), pa.binding.dtype_code(b.pk), partition,
        torch.cuda.current_stream().cuda_stream)
    return st


def _case(lens, partition, seed, kv_dtype="bf16", num_q_heads=32):
    w = make_workload(lens, num_q_heads=num_q_heads, num_kv_heads=8, head_dim=128, q_dtype="bf16", kv_dtype=kv_dtype,
                      seed=seed)
    b = DeviceBatch(w)
    need = pa.workspace_size(w.num_seqs, w.num_kv_heads, w.gqa_group, w.head_dim, w.max_context_len, partition)
    return w, b, need


def test_static_scratch_matches_caller_workspace_on_two_calls():
    # first call: a split whose partials take most of the array (P = 438 partitions of 16 tokens)
    w1, b1, need1 = _case([7000, 6001, 17, 1], 16, seed=71)
    assert 0.8 * LIMIT < need1 <= LIMIT, need1
    # second call, smaller: it reads only its own partials out of what the first call left
    w2, b2, need2 = _case([900, 1, 513, 0, 64], 64, seed=72)
    assert 0 < need2 < need1
    for tag, w, b, part in (("first", w1, b1, 16), ("second", w2, b2, 64)):
        print(f"[no-alloc] {tag} call: lens {w.context_lens.tolist()}, partition {part}", flush=True)
        got = torch.full_like(b.q, float("nan"))
        assert _static(b, part, got) == 0, pa.lib().pa_last_error().decode()
        ref = b.decode(part)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{tag} call differs"


def test_static_scratch_whole_context_and_e5m2():
    # partition 0 (no split, the array unused) and an automatic split over an E5M2 pool
    w, b, _ = _case([3000, 40, 2047], 0, seed=73, kv_dtype="e5m2")
    for part in (0, -1, 256):
        print(f"[no-alloc] e5m2 pool, partition {part}", flush=True)
        got = torch.empty_like(b.q)
        assert _static(b, part, got) == 0, pa.lib().pa_last_error().decode()
        ref = b.decode(part)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"partition {part} differs"


def test_static_scratch_on_the_matrix_core_decode_path():
    # 8 query heads per KV head: the partition pass runs on MFMA; a split call, then a smaller one
    # and a whole-context one on the same array
    for lens, part, seed in (([5000, 17, 1200], 64, 74), ([700, 1, 300], 256, 75), ([2100, 9], 0, 76)):
        w, b, need = _case(lens, part, seed=seed, num_q_heads=64)
        assert need <= LIMIT, need
        print(f"[no-alloc] G8 lens {w.context_lens.tolist()}, partition {part}", flush=True)
        got = torch.full_like(b.q, float("nan"))
        assert _static(b, part, got) == 0, pa.lib().pa_last_error().decode()
        ref = b.decode(part)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"G8 partition {part} differs"


def test_static_scratch_refuses_a_split_larger_than_the_array():
    # the host sizes the split by num_seqs and max_context_len: 4 x 32 heads x 1024 partitions
    w, b, _ = _case([300, 20, 5, 1], 16, seed=74)
    big = 16384
    need = pa.workspace_size(w.num_seqs, w.num_kv_heads, w.gqa_group, w.head_dim, big, 16)
    assert need > LIMIT
    got = torch.zeros_like(b.q)
    assert _static(b, 16, got, max_context_len=big) == 3  # PA_ERR_WORKSPACE_TOO_SMALL, nothing launched
    assert b"scratch" in pa.lib().pa_last_error()
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(got)) == 0
    # the python binding raises with the same status
    with pytest.raises(pa.PagedAttnError):
        pa.paged_attention_decode_static(b.q, b.pk, b.pv, b.tables, b.lens, big, w.scale, 16)
