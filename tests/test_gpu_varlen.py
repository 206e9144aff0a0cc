"""GPU parity of the packed (varlen) step against the float64 oracle (needs an MI355X).

Prefill rows (sequences with >= 2 new tokens) run on MFMA tiles, 1-token rows on the decode
kernel.  Bar: bf16 attention within 1e-2 absolute of the oracle (the oracle attends in
float64 on the exact cache values -- bf16, or E5M2 codes for an FP8 cache -- causal mask
aligned to the end of the context).
"""
import dataclasses
import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_251_amd as pa
from gpu_harness import DEV, DeviceBatch, assert_close, oracle_pools, out_f64, to_device
from workloads import make_config, make_workload, queries

pytestmark = pytest.mark.gpu


def _varlen(b: DeviceBatch, part=-1, causal=True, q=None, cu=None, lens=None, tables=None):
    w = b.w
    cu = torch.from_numpy(w.cu_seqlens_q).to(DEV) if cu is None else cu
    return pa.paged_attention_varlen(b.q if q is None else q, b.pk, b.pv, cu, b.lens if lens is None else lens,
                                     b.tables if tables is None else tables, w.max_q_len, w.max_context_len, w.scale,
                                     causal=causal, partition_size=part)


def _oracle_rows(w, pk, pv, causal=True):
    res = oracle.paged_varlen(pk, pv, w.kv_dtype, queries(w), w.q_dtype, w.cu_seqlens_q, w.block_tables,
                              w.context_lens, w.block_size, w.scale, causal=causal)
    return np.concatenate([res[s] for s in range(w.num_seqs)])


@pytest.mark.parametrize("kv", ["bf16", "e5m2"])
def test_varlen_workload_full_size(kv):
    w = dataclasses.replace(make_config(5), src_dtype="bf16", kv_dtype=kv)
    b = DeviceBatch(w)
    pk, pv = oracle_pools(w)
    ref = _oracle_rows(w, pk, pv)
    for part in (-1, 512):
        got = out_f64(_varlen(b, part), "bf16")
        err = assert_close(got, ref, "bf16", f"varlen {kv} partition {part}")
        print(f"varlen {kv} partition {part}: max abs err {err:.2e}")


def _mixed(seed, G, D, hkv=2, kv="bf16"):
    rng = np.random.default_rng(seed)
    n_new = [2, 3, 17, 31, 32, 33, 100, 1, 1, 64, 5, 1]
    cached = [0, 1, 15, 16, 100, 0, 7, 40, 0, 300, 2, 17]
    lens = np.array(cached) + np.array(n_new)
    order = rng.permutation(len(lens))
    return make_workload(lens[order], q_lens=np.array(n_new)[order], num_q_heads=hkv * G, num_kv_heads=hkv,
                         head_dim=D, q_dtype="bf16", src_dtype="bf16", kv_dtype=kv, seed=seed)


@pytest.mark.parametrize("G,D,causal,kv", [
    (4, 128, True, "bf16"), (1, 128, True, "bf16"), (2, 128, False, "bf16"), (8, 128, True, "bf16"),
    (16, 128, True, "bf16"), (4, 64, True, "bf16"), (8, 64, False, "bf16"), (16, 64, True, "bf16"),
    (4, 128, True, "e5m2"), (1, 128, True, "e5m2"), (2, 128, False, "e5m2"), (16, 128, True, "e5m2"),
    (8, 64, True, "e5m2"), (16, 64, False, "e5m2"),
])
def test_varlen_edge_lengths(G, D, causal, kv):
    w = _mixed(zlib.crc32(f"vl{G}{D}{causal}".encode()) % 1000, G, D, kv=kv)
    w.causal = causal
    b = DeviceBatch(w)
    pk, pv = oracle_pools(w)
    ref = _oracle_rows(w, pk, pv, causal)
    for part in (0, 16):
        assert_close(out_f64(_varlen(b, part, causal), "bf16"), ref, "bf16", f"varlen {kv} G{G} D{D} causal {causal}")


def test_varlen_more_sequences_than_the_ranked_limit():
    """Over 1024 sequences: both kernels fall back to their natural work order."""
    rng = np.random.default_rng(77)
    n_new = np.ones(1030, np.int64)
    n_new[[3, 500, 1029, 17, 800]] = [2, 33, 70, 5, 128]
    lens = n_new + rng.integers(0, 64, size=1030)
    w = make_workload(lens, q_lens=n_new, num_q_heads=4, num_kv_heads=2, head_dim=64, q_dtype="bf16", seed=77)
    b = DeviceBatch(w)
    pk, pv = oracle_pools(w)
    assert_close(out_f64(_varlen(b, 0), "bf16"), _oracle_rows(w, pk, pv), "bf16", "1030 sequences")


def test_varlen_packed_batch_above_the_one_launch_limit():
    """300 sequences with prefill chunks among them: above the two-role kernel's 256, the decode
    and prefill kernels run back to back, the decode rows in plain grid order (above 128)."""
    rng = np.random.default_rng(79)
    n_new = np.ones(300, np.int64)
    n_new[[0, 7, 150, 299]] = [40, 3, 129, 17]
    lens = n_new + rng.integers(0, 400, size=300)
    w = make_workload(lens, q_lens=n_new, num_q_heads=8, num_kv_heads=2, head_dim=128, q_dtype="bf16", seed=79)
    b = DeviceBatch(w)
    pk, pv = oracle_pools(w)
    assert_close(out_f64(_varlen(b, 0), "bf16"), _oracle_rows(w, pk, pv), "bf16", "300 sequences")


def test_varlen_block_permutation_and_packing_order_are_bit_identical():
    w = _mixed(5, 4, 128)
    b = DeviceBatch(w)
    base = _varlen(b, 0)
    # physical blocks moved
    rng = np.random.default_rng(3)
    perm = rng.permutation(w.num_blocks)
    inv = torch.from_numpy(np.argsort(perm)).to(DEV)
    pk2, pv2 = b.pk[inv].contiguous(), b.pv[inv].contiguous()
    bt2 = torch.from_numpy(np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)).to(DEV)
    cu = torch.from_numpy(w.cu_seqlens_q).to(DEV)
    moved = pa.paged_attention_varlen(b.q, pk2, pv2, cu, b.lens, bt2, w.max_q_len, w.max_context_len, w.scale,
                                      partition_size=0)
    assert torch.equal(base.view(torch.int16), moved.view(torch.int16))
    # sequences packed in reverse order
    order = np.arange(w.num_seqs)[::-1].copy()
    cu_np = w.cu_seqlens_q
    rows = np.concatenate([np.arange(cu_np[s], cu_np[s + 1]) for s in order])
    q_rev = b.q[torch.from_numpy(rows).to(DEV)].contiguous()
    cu_rev = torch.from_numpy(np.concatenate([[0], np.cumsum(w.q_lens[order])]).astype(np.int32)).to(DEV)
    rev = pa.paged_attention_varlen(q_rev, b.pk, b.pv, cu_rev, b.lens[torch.from_numpy(order).to(DEV)].contiguous(),
                                    b.tables[torch.from_numpy(order).to(DEV)].contiguous(), w.max_q_len,
                                    w.max_context_len, w.scale, partition_size=0)
    assert torch.equal(rev.view(torch.int16), base[torch.from_numpy(rows).to(DEV)].view(torch.int16))


def test_shared_prefix_equals_private_copy():
    from gpu_harness import poisoned_pool
    from workloads import seq_kv

    w = make_config(5)
    b = DeviceBatch(w)
    shared_out = _varlen(b, 0)
    # the same values with every sequence in private blocks
    priv = make_workload(w.context_lens, q_lens=w.q_lens, num_q_heads=32, num_kv_heads=8, head_dim=128,
                         q_dtype="bf16", seed=w.seed)
    tables = torch.from_numpy(priv.block_tables).to(DEV)
    pk, pv = poisoned_pool(priv), poisoned_pool(priv)
    for s in range(w.num_seqs):
        k, v = seq_kv(w, s)
        L = int(w.context_lens[s])
        cu = torch.tensor([0, L], dtype=torch.int32, device=DEV)
        end = torch.tensor([L], dtype=torch.int32, device=DEV)
        slots = pa.slot_mapping(cu, end, tables[s : s + 1].contiguous(), L, priv.num_blocks)
        pa.kv_cache_write(to_device(k, "bf16"), to_device(v, "bf16"), pk, pv, slots)
    private_out = pa.paged_attention_varlen(b.q, pk, pv, torch.from_numpy(w.cu_seqlens_q).to(DEV), b.lens, tables,
                                            w.max_q_len, w.max_context_len, w.scale, partition_size=0)
    assert torch.equal(shared_out.view(torch.int16), private_out.view(torch.int16))


@pytest.mark.parametrize("kv", ["bf16", "e5m2"])
def test_one_launch_equals_the_rows_called_apart(kv):
    """A packed step with both prefill chunks and decode tokens runs as one two-role launch; its
    output equals, bit for bit, the prefill chunks and the decode tokens each called on their own
    (the decode tokens then run on the plain decode kernel)."""
    w = dataclasses.replace(make_config(5), src_dtype="bf16", kv_dtype=kv)
    b = DeviceBatch(w)
    full = _varlen(b, 0)
    n_pre = int((w.q_lens > 1).sum())
    assert np.all(w.q_lens[:n_pre] > 1) and np.all(w.q_lens[n_pre:] == 1)  # chunks packed first
    rows = int(w.cu_seqlens_q[n_pre])
    cu = torch.from_numpy(w.cu_seqlens_q).to(DEV)
    pre = pa.paged_attention_varlen(b.q[:rows].contiguous(), b.pk, b.pv, cu[: n_pre + 1].contiguous(), b.lens[:n_pre],
                                    b.tables[:n_pre].contiguous(), w.max_q_len, w.max_context_len, w.scale,
                                    partition_size=0)
    dec = pa.paged_attention_varlen(b.q[rows:].contiguous(), b.pk, b.pv, (cu[n_pre:] - rows).contiguous(),
                                    b.lens[n_pre:].contiguous(), b.tables[n_pre:].contiguous(), 1, w.max_context_len,
                                    w.scale, partition_size=0)
    assert torch.equal(full[:rows].view(torch.int16), pre.view(torch.int16))
    assert torch.equal(full[rows:].view(torch.int16), dec.view(torch.int16))
