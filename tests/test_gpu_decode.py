"""GPU parity of the decode path against the float64 oracle (needs an MI355X).

Bars: slot mapping, cache writes and the E5M2 cast bit-exact; fp32 attention within
1e-5 of each output row's largest magnitude; bf16 attention within 1e-2 absolute;
E5M2-cache attention within 1e-2 absolute of the oracle run on the same E5M2 pool.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_251_amd as pa
from gpu_harness import (DEV, DeviceBatch, assert_close, canonical, oracle_pools, out_f64, poisoned_pool,
                         to_device)
from workloads import make_config, make_workload, queries

pytestmark = pytest.mark.gpu


def _oracle_decode(w, pk, pv, seqs=None):
    return oracle.paged_decode(pk, pv, w.kv_dtype, queries(w), w.q_dtype, w.block_tables, w.context_lens,
                               w.block_size, w.scale, seqs=seqs)


# ---------------------------------------------------------------- slot mapping / writes
@pytest.mark.parametrize("idx,phase", [(1, "all"), (2, "new"), (5, "all"), (5, "cached"), (5, "new")])
def test_slot_mapping_bit_exact(idx, phase):
    w = make_config(idx)
    b = DeviceBatch(w, phases=(phase,))
    plan, slots = b.slots[phase]
    want = oracle.slot_mapping(w.block_tables, plan.counts, plan.end_pos, w.block_size)
    assert np.array_equal(slots.cpu().numpy(), want)


def test_slot_mapping_out_of_range_rows_get_minus_one():
    tables = torch.tensor([[3, -1, 9], [0, 1, 2]], dtype=torch.int32, device=DEV)
    cu = torch.tensor([0, 4, 6], dtype=torch.int32, device=DEV)
    end = torch.tensor([40, 49], dtype=torch.int32, device=DEV)  # seq 1 runs past its 3 blocks
    got = pa.slot_mapping(cu, end, tables, 7, num_blocks=8).cpu().numpy()
    # seq 0: positions 36..39 -> logical block 2 -> entry 9 >= 8 blocks -> -1
    # seq 1: positions 47, 48 -> 47 in block 2 (phys 2, slot 47); 48 past the table -> -1
    # row 6 is not covered by cu -> -1
    assert got.tolist() == [-1, -1, -1, -1, 2 * 16 + 15, -1, -1]


@pytest.mark.parametrize("idx", [1, 2])
def test_cache_write_bit_exact_with_poison_kept(idx):
    w = make_config(idx)
    b = DeviceBatch(w)
    ok, ov = oracle_pools(w)
    assert np.array_equal(canonical(b.pk, w.kv_dtype).view(np.uint8), ok.view(np.uint8))
    assert np.array_equal(canonical(b.pv, w.kv_dtype).view(np.uint8), ov.view(np.uint8))


def test_e5m2_cast_bit_exact_on_every_bf16_pattern():
    patterns = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(64, 8, 128)
    w = make_workload([64], num_q_heads=8, num_kv_heads=8, head_dim=128, q_dtype="bf16", src_dtype="bf16",
                      kv_dtype="e5m2", pool=4, seed=1)
    pk = poisoned_pool(w)
    pv = poisoned_pool(w)
    slots = torch.arange(64, dtype=torch.int32, device=DEV)
    src = to_device(patterns, "bf16")
    pa.kv_cache_write(src, src, pk, pv, slots)
    got = canonical(pk, "e5m2").reshape(64, 8, 128)
    want = oracle.f64_to_e5m2(oracle.bf16_to_f64(patterns))
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, [(hex(int(patterns[i])), hex(int(got[i])), hex(int(want[i]))) for i in zip(*bad)][:8]
    assert np.array_equal(canonical(pv, "e5m2").reshape(64, 8, 128), want)


def test_cache_write_skips_negative_and_out_of_range_slots():
    w = make_workload([32], num_q_heads=2, num_kv_heads=2, head_dim=64, q_dtype="bf16", pool=2, seed=2)
    pk = poisoned_pool(w)
    pv = poisoned_pool(w)
    rows = to_device(np.full((4, 2, 64), 0x3F80, np.uint16), "bf16")  # 1.0
    slots = torch.tensor([-1, 5, 32, 1 << 20], dtype=torch.int32, device=DEV)
    pa.kv_cache_write(rows, rows, pk, pv, slots)
    got = canonical(pk, "bf16").reshape(32, 2, 64)
    assert np.all(got[5] == 0x3F80)
    others = np.delete(got, 5, axis=0)
    assert np.all(others == 0x7FC0)


# ---------------------------------------------------------------- decode
def test_tiny_fp32_decode_all_partitions():
    w = make_config(1)
    b = DeviceBatch(w)
    pk, pv = oracle_pools(w)
    ref = _oracle_decode(w, pk, pv)
    for part in (0, 16, 32, 64, -1):
        got = out_f64(b.decode(part), "f32")
        assert_close(got, ref, "f32", f"partition {part}")
        # context length 1: exactly that V row
        v0 = oracle.decode_storage(pv[w.block_tables[0, 0], 0], "f32")
        for h in range(4):
            assert np.array_equal(got[0, h], v0[h // 2])


def test_llama3_8b_bf16_decode_full_size():
    w = make_config(2)
    b = DeviceBatch(w)
    pk, pv = oracle_pools(w)
    ref = _oracle_decode(w, pk, pv)
    for part in (-1, 0, 512):
        err = assert_close(out_f64(b.decode(part), "bf16"), ref, "bf16", f"partition {part}")
        print(f"config 2 partition {part}: max abs err {err:.2e}")


@pytest.mark.parametrize("dtype,hkv,n", [("bf16", 3, 100), ("e5m2", 5, 230), ("bf16", 8, 40)])
def test_longest_first_order_covers_every_sequence_and_head(dtype, hkv, n):
    """Whole-context pass with more (sequence, KV head) units than CUs, a count that is not a
    multiple of the CU count, and many equal lengths: every unit is attended exactly once
    (the longest-first and snake orders only decide which work-group takes which unit)."""
    rng = np.random.default_rng(n)
    lens = rng.integers(0, 300, size=n)
    lens[::7] = 64  # ties
    w = make_workload(lens, num_q_heads=hkv * 2, num_kv_heads=hkv, head_dim=64, q_dtype="bf16",
                      kv_dtype=dtype, seed=n)
    b = DeviceBatch(w)
    pk, pv = oracle_pools(w)
    ref = _oracle_decode(w, pk, pv)
    assert_close(out_f64(b.decode(0), "bf16"), ref, "bf16", f"{dtype} {n}x{hkv} whole-context")


def _perm_pools(w, b: DeviceBatch, seed=5):
    rng = np.random.default_rng(seed)
    perm = rng.permutation(w.num_blocks)
    inv = torch.from_numpy(np.argsort(perm)).to(DEV)
    pk2 = b.pk[inv].contiguous()  # physical block x moves to perm[x]
    pv2 = b.pv[inv].contiguous()
    bt2 = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    return pk2, pv2, torch.from_numpy(bt2).to(DEV)


@pytest.mark.parametrize("idx", [1, 2])
def test_block_permutation_is_bit_identical(idx):
    w = make_config(idx)
    b = DeviceBatch(w)
    pk2, pv2, bt2 = _perm_pools(w, b)
    for part in (0, 256):
        base = b.decode(part)
        moved = pa.paged_attention_decode(b.q, pk2, pv2, bt2, b.lens, w.max_context_len, w.scale, partition_size=part)
        assert torch.equal(base.view(torch.int16 if w.q_dtype == "bf16" else torch.int32),
                           moved.view(torch.int16 if w.q_dtype == "bf16" else torch.int32))


# Per wave of a 4-wave whole-context pass these give 0 to 16 tiles: every peeled tail of the
# prefetch loop (100 and 150: two and three tiles on the first waves)
EDGE_LENS = [0, 1, 2, 15, 16, 17, 100, 150, 255, 256, 257, 511, 512, 513, 700, 1000]


@pytest.mark.parametrize("dtype,D,hkv,G", [
    ("bf16", 128, 2, 1), ("bf16", 128, 2, 2), ("bf16", 128, 1, 4), ("bf16", 128, 1, 8), ("bf16", 128, 1, 16),
    ("bf16", 64, 2, 4), ("bf16", 64, 1, 8), ("f32", 64, 2, 2), ("f32", 128, 1, 4), ("f32", 64, 1, 16),
    ("e5m2", 128, 2, 4), ("e5m2", 128, 1, 8), ("e5m2", 64, 2, 2), ("e5m2", 64, 1, 16),
])
def test_edge_lengths_gqa_and_head_dims(dtype, D, hkv, G):
    qd = "f32" if dtype == "f32" else "bf16"
    w = make_workload(EDGE_LENS, num_q_heads=hkv * G, num_kv_heads=hkv, head_dim=D, q_dtype=qd, src_dtype=qd,
                      kv_dtype=dtype, seed=zlib.crc32(f"{dtype}{D}{hkv}{G}".encode()) % 1000)
    b = DeviceBatch(w)
    pk, pv = oracle_pools(w)
    ref = _oracle_decode(w, pk, pv)
    for part in (0, 256, 512, -1):
        got = out_f64(b.decode(part), qd)
        assert_close(got, ref, qd, f"{dtype} D{D} G{G} partition {part}")
        assert np.all(got[0] == 0.0)  # empty context


def test_invalid_table_entries_are_skipped_without_fault():
    w = make_workload([40, 40], num_q_heads=4, num_kv_heads=2, head_dim=128, q_dtype="bf16", seed=9)
    b = DeviceBatch(w)
    good = b.decode(0).clone()
    bad_tables = b.tables.clone()
    bad_tables[1, 1] = -7
    bad_tables[1, 2] = 1 << 30
    out = pa.paged_attention_decode(b.q, b.pk, b.pv, bad_tables, b.lens, w.max_context_len, w.scale, partition_size=0)
    assert torch.equal(out[0].view(torch.int16), good[0].view(torch.int16))
    # sequence 1 now sees only its first block
    pk, pv = oracle_pools(w)
    ref = oracle.paged_decode(pk, pv, "bf16", queries(w)[1:2], "bf16", w.block_tables[1:2], np.array([16]), 16,
                              w.scale)
    assert_close(out_f64(out[1:2], "bf16"), ref, "bf16", "truncated sequence")
    # lengths beyond the table / negative lengths are clamped
    lens = torch.tensor([-3, 10 ** 6], dtype=torch.int32, device=DEV)
    out2 = pa.paged_attention_decode(b.q, b.pk, b.pv, b.tables, lens, w.max_context_len, w.scale, partition_size=16)
    assert torch.all(out2[0].float() == 0)
    assert torch.equal(out2[1].view(torch.int16), pa.paged_attention_decode(
        b.q, b.pk, b.pv, b.tables, b.lens, w.max_context_len, w.scale, partition_size=16)[1].view(torch.int16))


# ---------------------------------------------------------------- fused append + decode
def _append_case(w, part):
    from workloads import STORAGE, seq_kv

    a = DeviceBatch(w, phases=("cached",))
    b = DeviceBatch(w, phases=("cached",))
    # the newest row of every sequence ([N, Hkv, D]; zeros for an empty context, not read)
    kn = np.zeros((w.num_seqs, w.num_kv_heads, w.head_dim), STORAGE[w.src_dtype])
    vn = np.zeros_like(kn)
    for s in range(w.num_seqs):
        if w.context_lens[s] > 0:
            ks, vs = seq_kv(w, s)
            kn[s], vn[s] = ks[-1], vs[-1]
    k = to_device(kn, w.src_dtype)
    v = to_device(vn, w.src_dtype)
    a.write("new")
    out_sep = a.decode(part)
    out_fused = pa.paged_attention_decode_append(b.q, k, v, b.pk, b.pv, b.tables, b.lens, w.max_context_len,
                                                 w.scale, partition_size=part)
    return a, b, out_sep, out_fused


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32) if t.dtype == torch.float32 else t


@pytest.mark.parametrize("idx,part", [(1, 0), (1, 32), (2, -1), (2, 0), (2, 512)])
def test_append_is_bit_identical_to_write_then_decode(idx, part):
    w = make_config(idx)
    a, b, out_sep, out_fused = _append_case(w, part)
    assert torch.equal(_bits(out_sep), _bits(out_fused))
    assert torch.equal(_bits(a.pk), _bits(b.pk)) and torch.equal(_bits(a.pv), _bits(b.pv))


@pytest.mark.parametrize("dtype,D,G", [("e5m2", 128, 4), ("e5m2", 64, 8), ("bf16", 64, 2), ("f32", 128, 4),
                                         ("bf16", 128, 16), ("e5m2", 128, 8)])
def test_append_edge_lengths_against_oracle(dtype, D, G):
    qd = "f32" if dtype == "f32" else "bf16"
    w = make_workload([1, 2, 16, 17, 32, 33, 300, 513, 0], num_q_heads=2 * G, num_kv_heads=2, head_dim=D, q_dtype=qd,
                      src_dtype=qd, kv_dtype=dtype, seed=zlib.crc32(f"app{dtype}{D}{G}".encode()) % 1000)
    pk, pv = oracle_pools(w)
    ref = _oracle_decode(w, pk, pv)
    for part in (0, 256):
        a, b, out_sep, out_fused = _append_case(w, part)
        assert torch.equal(_bits(out_sep), _bits(out_fused))
        assert np.array_equal(canonical(b.pk, dtype).view(np.uint8), pk.view(np.uint8))
        assert np.array_equal(canonical(b.pv, dtype).view(np.uint8), pv.view(np.uint8))
        assert_close(out_f64(out_fused, qd), ref, qd, f"append {dtype} D{D} G{G} partition {part}")
