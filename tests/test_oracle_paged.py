"""Pins for the oracle's paged side: slot mapping, cache write, gather (CPU only).

Facts used (Colossal-Inference release post, section "分块式KV缓存
(BlockedKeyValueCache)"; LLM inference optimisation overview, section 2.1.2):
logical blocks map through a block table to physical blocks that need not be
contiguous; where a block lives does not change the result; memory is wasted
only in a sequence's last block; several logical blocks may share one
physical block (reference counting).  Section "KV缓存量化" of the release
post: an E5M2 cache takes half the memory of a 16-bit one.
"""
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import (attend, cache_write, decode_storage, gather_kv, new_pool, paged_decode,
                    paged_varlen, slot_mapping)
from workloads import POISON_BITS, make_config, make_workload, queries, seq_kv, write_plan


def _hand_slot_case():
    tables, writes, slots, bs = [], [], None, None
    with open(os.path.join(GOLDEN, "slot_mapping_hand.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            tag, *vals = line.split()
            if tag == "block_size":
                bs = int(vals[0])
            elif tag == "table":
                tables.append([int(x) for x in vals])
            elif tag == "write":
                writes.append((int(vals[0]), int(vals[1]), int(vals[2])))
            elif tag == "slots":
                slots = [int(x) for x in vals]
    counts = np.zeros(len(tables), np.int32)
    ends = np.zeros(len(tables), np.int32)
    for s, n, e in writes:
        counts[s], ends[s] = n, e
    return np.array(tables, np.int32), counts, ends, bs, np.array(slots)


def test_slot_mapping_hand_worked():
    bt, counts, ends, bs, want = _hand_slot_case()
    assert np.array_equal(slot_mapping(bt, counts, ends, bs), want)


def _build_pools(w, phase="all"):
    plan = write_plan(w, phase)
    slots = slot_mapping(w.block_tables, plan.counts, plan.end_pos, w.block_size)
    pk = new_pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.kv_dtype, POISON_BITS[w.kv_dtype])
    pv = new_pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.kv_dtype, POISON_BITS[w.kv_dtype])
    cache_write(pk, plan.k, slots, w.src_dtype, w.kv_dtype, w.block_size)
    cache_write(pv, plan.v, slots, w.src_dtype, w.kv_dtype, w.block_size)
    return pk, pv, slots


def _small_shared_workload(dtype="bf16"):
    lens = [130, 200, 16, 145, 300, 129]
    shared = [True, False, False, True, True, True]
    return make_workload(lens, num_q_heads=4, num_kv_heads=2, head_dim=16, q_dtype=dtype,
                         shared_seqs=shared, shared_prefix_blocks=8, seed=11)


def test_slots_are_a_bijection_except_intended_sharing():
    w = _small_shared_workload()
    owner = {}
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        sl = slot_mapping(w.block_tables, np.array([L if i == s else 0 for i in range(w.num_seqs)]),
                          w.context_lens, w.block_size)
        assert len(sl) == L
        assert len(set(sl.tolist())) == L  # distinct within a sequence
        for p, slot in enumerate(sl.tolist()):
            assert slot // w.block_size in w.block_tables[s, : -(-L // w.block_size)]
            if slot in owner:  # only the common prefix may be shared
                s0, p0 = owner[slot]
                assert w.shared_seqs[s] and w.shared_seqs[s0] and p == p0 < 128
            owner[slot] = (s, p)


def test_gather_reproduces_every_sequence_bit_exactly():
    for w in (_small_shared_workload("bf16"), _small_shared_workload("f32")):
        pk, pv, _ = _build_pools(w)
        for s in range(w.num_seqs):
            k, v = seq_kv(w, s)
            L = int(w.context_lens[s])
            assert np.array_equal(gather_kv(pk, w.block_tables[s], L, w.block_size), k)
            assert np.array_equal(gather_kv(pv, w.block_tables[s], L, w.block_size), v)


def test_waste_only_in_last_block_and_tail_keeps_poison():
    w = make_config(1)
    pk, pv, slots = _build_pools(w)
    used = set()
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        nblk = -(-L // w.block_size)
        assert np.all(w.block_tables[s, nblk:] == -1)
        used.update(w.block_tables[s, :nblk].tolist())
        # only the last block has unwritten slots, and they still hold the poison
        last = w.block_tables[s, nblk - 1]
        tail = L - (nblk - 1) * w.block_size
        assert np.all(np.isnan(pk[last, tail:])) and np.all(np.isnan(pv[last, tail:]))
        assert not np.any(np.isnan(pk[last, :tail]))
    assert len(slots) == int(w.context_lens.sum())
    assert len(used) == sum(-(-int(L) // 16) for L in w.context_lens)
    spare = [b for b in range(w.num_blocks) if b not in used]
    assert np.all(np.isnan(pk[spare]))


def test_physical_block_permutation_leaves_output_bit_identical():
    w = make_config(1)
    pk, pv, _ = _build_pools(w)
    q = queries(w)
    base = paged_decode(pk, pv, w.kv_dtype, q, w.q_dtype, w.block_tables, w.context_lens, w.block_size, w.scale)
    rng = np.random.default_rng(9)
    perm = rng.permutation(w.num_blocks)  # physical block b moves to perm[b]
    pk2 = np.empty_like(pk)
    pv2 = np.empty_like(pv)
    pk2[perm] = pk
    pv2[perm] = pv
    bt2 = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1)
    out = paged_decode(pk2, pv2, w.kv_dtype, q, w.q_dtype, bt2, w.context_lens, w.block_size, w.scale)
    assert np.array_equal(out, base)
    assert np.all(np.isfinite(out))


def test_paged_decode_equals_contiguous_attention():
    w = make_config(1)
    pk, pv, _ = _build_pools(w)
    q = queries(w)
    out = paged_decode(pk, pv, w.kv_dtype, q, w.q_dtype, w.block_tables, w.context_lens, w.block_size, w.scale)
    qd = decode_storage(q, w.q_dtype)
    for s in range(w.num_seqs):
        k, v = seq_kv(w, s)
        ref = attend(qd[s : s + 1], decode_storage(k, "f32"), decode_storage(v, "f32"), 1 / 8)
        assert np.array_equal(out[s], ref[0])
    # context length 1: the single V row, exactly
    k0, v0 = seq_kv(w, 0)
    for h in range(4):
        assert np.array_equal(out[0, h], decode_storage(v0, "f32")[0, h // 2])


def test_shared_prefix_equals_private_copy():
    w = _small_shared_workload()
    pk, pv, _ = _build_pools(w)
    q = queries(w)
    shared_out = paged_decode(pk, pv, "bf16", q, "bf16", w.block_tables, w.context_lens, 16, w.scale)
    # same data with the common prefix copied into private blocks
    private = make_workload(w.context_lens, num_q_heads=4, num_kv_heads=2, head_dim=16, q_dtype="bf16", seed=11)
    pk2 = new_pool(private.num_blocks, 16, 2, 16, "bf16", POISON_BITS["bf16"])
    pv2 = new_pool(private.num_blocks, 16, 2, 16, "bf16", POISON_BITS["bf16"])
    for s in range(w.num_seqs):
        k, v = seq_kv(w, s)
        L = int(w.context_lens[s])
        counts = np.array([L if i == s else 0 for i in range(w.num_seqs)])
        sl = slot_mapping(private.block_tables, counts, private.context_lens, 16)
        cache_write(pk2, k, sl, "bf16", "bf16", 16)
        cache_write(pv2, v, sl, "bf16", "bf16", 16)
    priv_out = paged_decode(pk2, pv2, "bf16", q, "bf16", private.block_tables, w.context_lens, 16, w.scale)
    assert np.array_equal(shared_out, priv_out)
    # prefix blocks are physically common to every sharing sequence
    common = w.block_tables[w.shared_seqs][:, :8]
    assert np.all(common == common[0])


def test_e5m2_pool_is_half_of_bf16_and_decodes_to_nearest():
    w = make_workload([40, 5], num_q_heads=2, num_kv_heads=1, head_dim=16, q_dtype="bf16",
                      src_dtype="bf16", kv_dtype="e5m2", seed=3)
    pk, pv, _ = _build_pools(w)
    pool16 = new_pool(w.num_blocks, 16, 1, 16, "bf16", 0)
    assert pk.nbytes * 2 == pool16.nbytes
    k, _ = seq_kv(w, 0)
    got = decode_storage(gather_kv(pk, w.block_tables[0], 40, 16), "e5m2")
    exact = decode_storage(k, "bf16")
    # |x - e5m2(x)| <= half an e5m2 ulp: 2^-3 relative for normal values
    big = np.abs(exact) >= 2.0**-14
    assert np.all(np.abs(got[big] - exact[big]) <= np.abs(exact[big]) * 2.0**-3)


def test_varlen_history_plus_new_equals_full_write():
    w = _small_shared_workload()
    w.q_lens = np.array([2, 5, 1, 1, 7, 1], np.int32)
    pk, pv, _ = _build_pools(w, "all")
    pk2, pv2, _ = _build_pools(w, "cached")
    plan = write_plan(w, "new")
    sl = slot_mapping(w.block_tables, plan.counts, plan.end_pos, 16)
    cache_write(pk2, plan.k, sl, "bf16", "bf16", 16)
    cache_write(pv2, plan.v, sl, "bf16", "bf16", 16)
    assert np.array_equal(pk.view(np.uint16), pk2.view(np.uint16))
    q = queries(w)
    res = paged_varlen(pk, pv, "bf16", q, "bf16", w.cu_seqlens_q, w.block_tables, w.context_lens, 16, w.scale)
    # last query of each sequence = decode of that sequence
    qd = decode_storage(q, "bf16")
    for s, o in res.items():
        k, v = seq_kv(w, s)
        ref = attend(qd[w.cu_seqlens_q[s + 1] - 1 : w.cu_seqlens_q[s + 1]], decode_storage(k, "bf16"),
                     decode_storage(v, "bf16"), w.scale)
        np.testing.assert_allclose(o[-1:], ref, rtol=0, atol=1e-14)
    # packing order does not matter: reversing the sequences gives the same rows
    order = np.arange(w.num_seqs)[::-1]
    qd_rev = np.concatenate([q[w.cu_seqlens_q[s] : w.cu_seqlens_q[s + 1]] for s in order])
    cu_rev = np.concatenate([[0], np.cumsum(w.q_lens[order])])
    res_rev = paged_varlen(pk, pv, "bf16", qd_rev, "bf16", cu_rev, w.block_tables[order], w.context_lens[order],
                           16, w.scale)
    for i, s in enumerate(order):
        assert np.array_equal(res_rev[i], res[s])


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_config_shapes(idx):
    w = make_config(idx)
    need = sum(-(-int(L) // 16) for L in w.context_lens)
    if idx == 1:
        assert list(w.context_lens) == [1, 17, 33, 100] and w.num_blocks == 32 and w.q_dtype == "f32"
    if idx == 2:
        assert w.num_seqs == 64 and (w.num_q_heads, w.num_kv_heads, w.head_dim) == (32, 8, 128)
        assert w.context_lens.min() >= 512 and w.context_lens.max() <= 2048
        assert w.num_blocks == (11 * need + 9) // 10
    if idx == 3:
        assert w.num_seqs == 128 and w.kv_dtype == "e5m2" and w.src_dtype == "bf16"
        assert w.context_lens.min() >= 256 and w.context_lens.max() <= 4096
    if idx == 4:
        assert np.all(w.context_lens == 32768) and w.num_q_heads == 64 and w.partition_size == 512
    if idx == 5:
        assert w.num_seqs == 132 and w.total_q == int(w.q_lens[:4].sum()) + 128
        assert np.all(w.q_lens[4:] == 1) and np.all((w.q_lens[:4] >= 256) & (w.q_lens[:4] <= 1024))
        cached = w.context_lens[:4] - w.q_lens[:4]
        assert np.all((cached >= 0) & (cached <= 2048))
        assert int(w.shared_seqs.sum()) == 33
        assert np.all(w.context_lens[w.shared_seqs] - w.q_lens[w.shared_seqs] >= 128)
        unique = need - 32 * 8
        assert w.num_blocks == (11 * unique + 9) // 10
    used = w.block_tables[w.block_tables >= 0]
    assert used.max() < w.num_blocks
