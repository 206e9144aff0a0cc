"""Query elements at the edge of f16's range over the 8-bit caches (needs an MI355X).

Over an FP8_E5M2, INT8 or FP8_E4M3 cache the kernels take the bf16 query to f16 for the dot
products.  That is exact for bf16 values of magnitude 2^-14 .. 65280 (the largest bf16 value
below f16's overflow), so rows whose elements reach 65280 must match the oracle, which uses the
bf16 query as it is.  An element of magnitude 65536 or more is outside the supported range: the
header leaves the output row of its (sequence, head) unspecified and states that no other head or
sequence is affected, which is what is checked.  Both for the decode calls and for packed batches
(prefill tiles and the multi-token kernel).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_251_amd as pa
from gpu_harness import DEV, DeviceBatch, assert_close, oracle_int8_pools, oracle_pools, out_f64, to_device
from workloads import make_workload, queries

pytestmark = pytest.mark.gpu

BF16_65280 = 0x477F  # 65280: the largest bf16 value that f16 holds
BF16_65536 = 0x4780  # 65536: rounds to inf in f16


def _big_queries(w):
    """The workload's queries scaled so that every row's largest element is +-65280 exactly; and
    the same with one element of (row 0, head 0) raised to 65536."""
    q = oracle.decode_storage(queries(w), "bf16")
    big = q * (65280.0 / np.abs(q).max(axis=-1, keepdims=True))
    raw = torch.from_numpy(np.ascontiguousarray(big, np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    raw = raw.view(np.uint16).copy()
    top = np.abs(big).argmax(axis=-1)
    rows, heads = np.indices(top.shape)
    raw[rows, heads, top] = np.where(big[rows, heads, top] > 0, BF16_65280, BF16_65280 | 0x8000)
    assert np.abs(oracle.decode_storage(raw, "bf16")).max() == 65280.0
    over = raw.copy()
    over[0, 0, 3] = BF16_65536
    return raw, over


def _ref_pools(w):
    if w.kv_dtype in ("int8", "e4m3"):
        o = oracle_int8_pools(w)
        return o["k"][3], o["v"][3], "f64"
    pk, pv = oracle_pools(w)
    return pk, pv, w.kv_dtype


@pytest.mark.parametrize("kind", ["e5m2", "int8", "e4m3"])
def test_decode_query_at_f16_edge(kind):
    w = make_workload([700, 1, 33, 2049], num_q_heads=16, num_kv_heads=4, head_dim=128, q_dtype="bf16",
                      src_dtype="bf16", kv_dtype=kind, seed=91)
    b = DeviceBatch(w)
    pk, pv, dt = _ref_pools(w)
    raw, over = _big_queries(w)
    scale = w.scale / 65280.0 * 4.0  # scores of a few units: the softmax is not one-hot
    ref = oracle.paged_decode(pk, pv, dt, raw, "bf16", w.block_tables, w.context_lens, 16, scale)
    for part in (0, 256):
        got = out_f64(pa.paged_attention_decode(to_device(raw, "bf16"), b.pk, b.pv, b.tables, b.lens,
                                                w.max_context_len, scale, partition_size=part), "bf16")
        err = assert_close(got, ref, "bf16", f"{kind} |q| up to 65280, partition {part}")
        print(f"{kind} partition {part}: max abs err {err:.2e}")
        got = out_f64(pa.paged_attention_decode(to_device(over, "bf16"), b.pk, b.pv, b.tables, b.lens,
                                                w.max_context_len, scale, partition_size=part), "bf16")
        keep = np.ones(got.shape[:2], bool)
        keep[0, 0] = False
        assert_close(got[keep], ref[keep], "bf16", f"{kind} other heads, partition {part}")


@pytest.mark.parametrize("q_lens", [[40, 1, 300, 2], [4, 4, 4, 4]])
def test_packed_query_at_f16_edge(q_lens):
    """Prefill tiles (chunks of 40 and 300 rows) and the multi-token kernel (4 rows each) over an
    E5M2 cache."""
    lens = np.array([100, 57, 900, 6]) + np.array(q_lens)
    w = make_workload(lens, q_lens=q_lens, num_q_heads=16, num_kv_heads=4, head_dim=128, q_dtype="bf16",
                      src_dtype="bf16", kv_dtype="e5m2", seed=92)
    b = DeviceBatch(w)
    pk, pv = oracle_pools(w)
    raw, over = _big_queries(w)
    scale = w.scale / 65280.0 * 4.0
    res = oracle.paged_varlen(pk, pv, "e5m2", raw, "bf16", w.cu_seqlens_q, w.block_tables, w.context_lens, 16, scale)
    ref = np.concatenate([res[s] for s in range(w.num_seqs)])
    cu = torch.from_numpy(w.cu_seqlens_q).to(DEV)
    for q, tag in ((raw, "edge"), (over, "over")):
        got = out_f64(pa.paged_attention_varlen(to_device(q, "bf16"), b.pk, b.pv, cu, b.lens, b.tables, w.max_q_len,
                                                w.max_context_len, scale), "bf16")
        if tag == "edge":
            err = assert_close(got, ref, "bf16", f"packed {q_lens} |q| up to 65280")
            print(f"packed {q_lens}: max abs err {err:.2e}")
        else:
            keep = np.ones(got.shape[:2], bool)
            keep[0, 0] = False
            assert_close(got[keep], ref[keep], "bf16", f"packed {q_lens} other rows")
