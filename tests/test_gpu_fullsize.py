"""Full-size parity of every sequence (needs an MI355X).

The Llama-3-8B E5M2 decode workload (128 sequences up to 4096 tokens) and the long-context
split-KV workload (8 x 32768 tokens, 512-token partitions) are written and attended on the
GPU at their real sizes, in the launch configurations bench.py times, and every output row is
compared with the float64 oracle run on the same pools.  The whole E5M2 pools are compared byte
for byte with the oracle's cast.  The split-KV partials left in the workspace are checked against
the oracle's per-partition softmax state, independently of the reduce kernel.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_251_amd as pa
from gpu_harness import DEV, DeviceBatch, assert_close, canonical, oracle_pools, oracle_pools_from_plan, out_f64
from workloads import make_config, make_workload, queries, write_plan

pytestmark = pytest.mark.gpu


def _full_batch(w):
    """The workload written on the GPU by the library and on the CPU by the oracle, from one plan."""
    plan = write_plan(w, "all")
    b = DeviceBatch(w, phases=())
    b.write("all", plan=plan)
    pk, pv = oracle_pools_from_plan(w, plan)
    return b, pk, pv


def test_e5m2_decode_full_size_every_sequence():
    w = make_config(3)
    b, pk, pv = _full_batch(w)
    # the whole pools, written slots and poisoned spares alike: bit-exact E5M2 cast
    assert np.array_equal(canonical(b.pk, "e5m2"), pk)
    assert np.array_equal(canonical(b.pv, "e5m2"), pv)
    ref = oracle.paged_decode(pk, pv, "e5m2", queries(w), "bf16", w.block_tables, w.context_lens, 16, w.scale)
    for part in (-1, 512):
        out = out_f64(b.decode(part), "bf16")
        err = assert_close(out, ref, "bf16", f"e5m2 full size partition {part}")
        print(f"e5m2 full size, all {w.num_seqs} sequences, partition {part}: max abs err {err:.2e}")


def test_long_context_split_kv_full_size_every_sequence():
    w = make_config(4)
    b, pk, pv = _full_batch(w)
    ref = oracle.paged_decode(pk, pv, "bf16", queries(w), "bf16", w.block_tables, w.context_lens, 16, w.scale)
    part = w.partition_size
    need = pa.workspace_size(w.num_seqs, w.num_kv_heads, w.gqa_group, w.head_dim, w.max_context_len, part)
    ws = pa.alloc_workspace(need, DEV)
    out = pa.paged_attention_decode(b.q, b.pk, b.pv, b.tables, b.lens, w.max_context_len, w.scale,
                                    partition_size=part, workspace=ws)
    err = assert_close(out_f64(out, "bf16"), ref, "bf16", "long context split-KV")
    print(f"long context, all {w.num_seqs} sequences: max abs err {err:.2e}")
    # the partials: o [N][Hq][P][D], m [N][Hq][P], l [N][Hq][P], each region 256-byte aligned
    n, hq, d = w.num_seqs, w.num_q_heads, w.head_dim
    P = -(-w.max_context_len // part)
    rnd = lambda x: (x + 255) // 256 * 256
    ob, mb = rnd(n * hq * P * d * 4), rnd(n * hq * P * 4)
    wsf = ws.view(torch.uint8)
    o = wsf[:ob].view(torch.float32)[: n * hq * P * d].view(n, hq, P, d).cpu().numpy().astype(np.float64)
    m = wsf[ob : ob + mb].view(torch.float32)[: n * hq * P].view(n, hq, P).cpu().numpy().astype(np.float64)
    l = wsf[ob + mb : ob + 2 * mb].view(torch.float32)[: n * hq * P].view(n, hq, P).cpu().numpy().astype(np.float64)
    qd = oracle.decode_storage(queries(w), "bf16")
    # With 8 query heads per KV head the partition pass runs on MFMA: its probabilities enter the
    # PV product and the row sum rounded to bf16 (unit roundoff u = 2^-9), the same rounded values
    # in both.  Each weight's relative error is then at most u, so the sum's is too (lse off by at
    # most -log2(1 - u)), and the normalised o moves by at most u / (1 - u) times the spread
    # (max - min) of the values it averages.  The vector pass keeps them in fp32 (u = 0 here).
    u = 2.0 ** -9 if w.gqa_group in (8, 16) else 0.0
    lse_tol = -np.log2(1 - u)
    for s in range(n):
        L = int(w.context_lens[s])
        kk = oracle.decode_storage(oracle.gather_kv(pk, w.block_tables[s], L, 16), "bf16")
        vv = oracle.decode_storage(oracle.gather_kv(pv, w.block_tables[s], L, 16), "bf16")
        om, ol, oo = oracle.attend_partitioned(qd[s : s + 1], kk, vv, w.scale, part)
        # The kernel keeps its running max in base 2 and rescales only when the max grows by more
        # than a fixed threshold, so the stored m may lag the true maximum; what is fixed is the
        # log-sum-exp m + log2(l) and the normalised o.
        lse_ref = (om[:, 0, :].T + np.log(ol[:, 0, :].T)) * np.log2(np.e)
        np.testing.assert_allclose(m[s] + np.log2(l[s]), lse_ref, rtol=0, atol=1e-4 + lse_tol)
        assert np.all(m[s] <= om[:, 0, :].T * np.log2(np.e) + 1e-4)
        # per partition and dim: u / (1 - u) times the spread of that partition's values
        ptp = np.stack([np.stack([np.ptp(vv[j * part : (j + 1) * part, h], axis=0) for j in range(P)])
                        for h in range(w.num_kv_heads)])  # [Hkv][P][D]
        bound = 1e-4 + u / (1 - u) * np.repeat(ptp, w.gqa_group, axis=0)  # [Hq][P][D]
        err = np.abs(o[s] - oo[:, 0].transpose(1, 0, 2))
        assert np.all(err <= bound), f"sequence {s} partials: max err {err.max():.2e}"


def test_context_of_128k_tokens():
    """One sequence of 131072 tokens (8192 blocks, 8 KV heads, 64 query heads) stored in the top
    of a 2.5 GB pool, so tile byte offsets pass 2^31: the automatic split (256 partitions of
    512) and a whole-context pass.  The oracle reads the same rows from a compact pool."""
    import dataclasses

    L = 131072
    w = make_workload([L, 5], num_q_heads=64, num_kv_heads=8, head_dim=128, q_dtype="bf16", seed=131)
    off = 66000  # (66000 + 9013 blocks) x 32 KiB per block = 2.46 GB per pool
    big = dataclasses.replace(w, block_tables=np.where(w.block_tables >= 0, w.block_tables + off, -1).astype(np.int32),
                              num_blocks=w.num_blocks + off)
    assert int(big.block_tables.max()) * 8 * 16 * 128 * 2 > 2**31
    b = DeviceBatch(big)
    pk, pv = oracle_pools(w)
    ref = oracle.paged_decode(pk, pv, "bf16", queries(w), "bf16", w.block_tables, w.context_lens, 16, w.scale)
    assert pa.auto_partition(w.num_seqs, w.num_kv_heads, w.gqa_group, w.head_dim, w.max_context_len) > 0
    for part in (-1, 0):
        err = assert_close(out_f64(b.decode(part), "bf16"), ref, "bf16", f"128k context, partition {part}")
        print(f"128k context partition {part}: max abs err {err:.2e}")
