"""GPU parity of multi-token decode (speculative verification) against the float64 oracle.

Every sequence of the batch attends k new tokens at once, causal among them, through
paged_attention_varlen (needs an MI355X).  When every sequence has exactly max_q_len >= 2 rows
the library launches only the MFMA tile kernel; a batch that mixes k and 1 also runs the
decode kernel.  Bar: bf16 within 1e-2 absolute of the oracle.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_251_amd as pa
from gpu_harness import DEV, DeviceBatch, assert_close, oracle_pools, out_f64
from workloads import make_config, make_workload, queries

pytestmark = pytest.mark.gpu


def _run(b: DeviceBatch, part=-1, causal=True):
    w = b.w
    cu = torch.from_numpy(w.cu_seqlens_q).to(DEV)
    return pa.paged_attention_varlen(b.q, b.pk, b.pv, cu, b.lens, b.tables, w.max_q_len, w.max_context_len, w.scale,
                                     causal=causal, partition_size=part)


def _oracle(w, pk, pv, causal=True):
    res = oracle.paged_varlen(pk, pv, w.kv_dtype, queries(w), w.q_dtype, w.cu_seqlens_q, w.block_tables,
                              w.context_lens, w.block_size, w.scale, causal=causal)
    return np.concatenate([res[s] for s in range(w.num_seqs)])


def test_spec_verify_workload_full_size():
    w = make_config(6)
    b = DeviceBatch(w)
    pk, pv = oracle_pools(w)
    err = assert_close(out_f64(_run(b), "bf16"), _oracle(w, pk, pv), "bf16", "speculative verification, k = 4")
    print(f"spec verify k=4: max abs err {err:.2e}")


@pytest.mark.parametrize("k,G,D,kv", [(2, 4, 128, "bf16"), (3, 8, 128, "bf16"), (5, 1, 128, "bf16"), (8, 4, 64, "bf16"),
                                      (16, 2, 64, "bf16"), (4, 16, 128, "bf16"), (4, 4, 128, "e5m2"),
                                      (3, 8, 128, "e5m2"), (16, 2, 64, "e5m2")])
def test_spec_verify_draft_lengths(k, G, D, kv):
    rng = np.random.default_rng(zlib.crc32(f"spec{k}{G}{D}".encode()))
    cached = np.array([0, 1, 15, 16, 17, 31, 64, 100, 255, 1000])
    lens = cached + k
    w = make_workload(lens[rng.permutation(len(lens))], q_lens=np.full(len(lens), k), num_q_heads=2 * G,
                      num_kv_heads=2, head_dim=D, q_dtype="bf16", src_dtype="bf16", kv_dtype=kv, seed=k * 100 + G)
    b = DeviceBatch(w)
    pk, pv = oracle_pools(w)
    ref = _oracle(w, pk, pv)
    for part in (0, 16):
        assert_close(out_f64(_run(b, part), "bf16"), ref, "bf16", f"k={k} G={G} D={D} {kv} partition {part}")


def test_mixed_draft_lengths_run_both_kernels():
    # one sequence verifies a single token: the batch is no longer uniform, the decode kernel runs too
    q_lens = np.array([4, 4, 1, 4, 3, 4])
    lens = np.array([40, 300, 77, 16, 5, 4])
    w = make_workload(lens, q_lens=q_lens, num_q_heads=8, num_kv_heads=2, head_dim=128, q_dtype="bf16", seed=606)
    b = DeviceBatch(w)
    pk, pv = oracle_pools(w)
    assert_close(out_f64(_run(b), "bf16"), _oracle(w, pk, pv), "bf16", "mixed draft lengths")


def test_uniform_batch_matches_its_split_into_halves():
    """The uniform batch (no decode launch) gives the same rows as the same sequences run in two
    calls of three; every row is computed by the same kernel either way, so bit-identical."""
    w = make_workload(np.array([100, 20, 513, 64, 9, 1000]), q_lens=np.full(6, 4), num_q_heads=32, num_kv_heads=8,
                      head_dim=128, q_dtype="bf16", seed=707)
    b = DeviceBatch(w)
    whole = _run(b, 0)
    parts = []
    for s0, s1 in ((0, 3), (3, 6)):
        cu = torch.from_numpy((w.cu_seqlens_q[s0 : s1 + 1] - w.cu_seqlens_q[s0]).astype(np.int32)).to(DEV)
        r0, r1 = int(w.cu_seqlens_q[s0]), int(w.cu_seqlens_q[s1])
        parts.append(pa.paged_attention_varlen(b.q[r0:r1].contiguous(), b.pk, b.pv, cu, b.lens[s0:s1].contiguous(),
                                               b.tables[s0:s1].contiguous(), 4, w.max_context_len, w.scale,
                                               partition_size=0))
    assert torch.equal(whole.view(torch.int16), torch.cat(parts).view(torch.int16))
