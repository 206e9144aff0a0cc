"""Seeded generators for the five paged-attention workloads and for small custom cases.

Storage conventions (raw bits, as they sit in device memory):
  'f32'  -> np.float32
  'bf16' -> np.uint16 bit patterns
  'e5m2' -> np.uint8 codes (only ever a cache dtype: the cast is done by the
            code under test, never here)
  'int8' -> int8 codes with a float32 scale per (token, KV head) row (a cache dtype
            only, like 'e5m2')
  'e4m3' -> FP8 E4M3 codes with a float32 scale per row (a cache dtype only)

Every random draw comes from ``np.random.default_rng([seed, stream, ...])`` so
that one sequence's keys and values can be regenerated on their own, which
lets the oracle check sampled sequences of a full-size workload without
materialising the rest.  Values are float32 N(0,1) draws rounded to the
storage dtype (bf16 by torch's round-to-nearest-even cast).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

STORAGE = {"f32": np.float32, "bf16": np.uint16, "e5m2": np.uint8}
ITEMSIZE = {"f32": 4, "bf16": 2, "e5m2": 1, "int8": 1, "e4m3": 1}
# bytes a pool stores per (token, KV head) row besides its head_dim elements
ROW_EXTRA = {"f32": 0, "bf16": 0, "e5m2": 0, "int8": 4, "e4m3": 4}

# Quiet-NaN patterns written over a pool before any cache write: a read of a
# slot that was never written (the tail of a last block, a spare block) then
# turns the output into NaN instead of going unnoticed.
POISON_BITS = {"f32": 0x7FC00000, "bf16": 0x7FC0, "e5m2": 0x7F,
               "int8": 0x7FC00000, "e4m3": 0x7FC00000}  # scaled pools: every 32-bit word, so every scale is NaN

CONFIG_NAMES = {
    1: "tiny_decode_fp32",
    2: "llama3_8b_decode_bf16",
    3: "llama3_8b_decode_e5m2_kv",
    4: "long_context_split_kv_bf16",
    5: "varlen_prefill_decode_bf16",
    6: "llama3_8b_spec_verify_k4_bf16",
    7: "llama3_8b_decode_int8_kv",
    8: "llama3_8b_decode_fp8_e4m3_scaled_kv",
    9: "varlen_prefill_decode_e5m2_kv",
}

# random streams
_S_LENS, _S_PERM, _S_SHARE, _S_Q, _S_KV, _S_SHARED_KV = 1, 2, 3, 4, 5, 6


@dataclass
class Workload:
    """One batch of sequences over a blocked KV pool (host arrays only)."""

    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_dtype: str
    src_dtype: str  # dtype of the K/V rows handed to the cache write
    kv_dtype: str  # dtype of the cache pools
    context_lens: np.ndarray  # int32 [N]: tokens in the context, current ones included
    q_lens: np.ndarray  # int32 [N]: query (new) tokens per sequence, 1 for decode
    block_tables: np.ndarray  # int32 [N, max_blocks]; -1 past a sequence's last block
    num_blocks: int  # physical blocks in the pool
    shared_seqs: np.ndarray  # bool [N]: sequence maps the common prefix blocks
    shared_prefix_blocks: int  # leading logical blocks that sharing sequences have in common
    partition_size: int  # split-KV partition (tokens) the workload asks for; 0 = none named
    causal: bool

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def gqa_group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def cu_seqlens_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def is_decode(self) -> bool:
        return bool(np.all(self.q_lens == 1))

    def kv_token_count(self) -> int:
        return int(self.context_lens.astype(np.int64).sum())


@dataclass
class WritePlan:
    """Token rows for one cache write.

    Sequence s contributes ``counts[s]`` rows, packed in sequence order; they
    belong at logical positions ``end_pos[s] - counts[s] .. end_pos[s] - 1``.
    """

    counts: np.ndarray  # int32 [N]
    end_pos: np.ndarray  # int32 [N]
    k: np.ndarray  # [T, Hkv, D] raw src dtype
    v: np.ndarray

    @property
    def cu(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.counts)]).astype(np.int32)

    @property
    def num_tokens(self) -> int:
        return int(self.counts.sum())


def _to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(f"values are generated as f32 or bf16, not {dtype}")


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return _to_storage(rng.standard_normal(size=shape, dtype=np.float32), dtype)


def _blocks_needed(lens: np.ndarray, block_size: int) -> np.ndarray:
    return (lens.astype(np.int64) + block_size - 1) // block_size


def _assign_blocks(rng, lens, block_size, shared, shared_blocks, pool=None):
    """Hand out physical block ids, taken in order from a seeded permutation."""
    need = _blocks_needed(lens, block_size)
    n_shared = int(shared.sum())
    unique = int(need.sum()) - (max(n_shared - 1, 0) * shared_blocks)
    if pool is None:
        pool = (11 * unique + 9) // 10  # +10 % spare blocks, rounded up
    if pool < unique:
        raise ValueError(f"pool of {pool} blocks cannot hold {unique}")
    perm = rng.permutation(pool).astype(np.int32)
    width = max(int(need.max()) if len(need) else 1, 1)
    tables = np.full((len(lens), width), -1, dtype=np.int32)
    nxt = 0
    common = None
    for s in range(len(lens)):
        for j in range(int(need[s])):
            if shared[s] and j < shared_blocks:
                if common is None:
                    common = perm[nxt : nxt + shared_blocks].copy()
                    nxt += shared_blocks
                tables[s, j] = common[j]
            else:
                tables[s, j] = perm[nxt]
                nxt += 1
    return tables, pool


def make_workload(
    context_lens,
    *,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int = 16,
    q_dtype: str = "bf16",
    src_dtype: str | None = None,
    kv_dtype: str | None = None,
    q_lens=None,
    pool: int | None = None,
    shared_seqs=None,
    shared_prefix_blocks: int = 0,
    partition_size: int = 0,
    causal: bool = True,
    seed: int = 0,
    name: str = "custom",
) -> Workload:
    lens = np.asarray(context_lens, dtype=np.int32).reshape(-1)
    n = lens.shape[0]
    qlens = np.ones(n, np.int32) if q_lens is None else np.asarray(q_lens, np.int32).reshape(-1)
    src_dtype = src_dtype or q_dtype
    kv_dtype = kv_dtype or src_dtype
    shared = np.zeros(n, bool) if shared_seqs is None else np.asarray(shared_seqs, bool)
    if shared_prefix_blocks == 0:
        shared = np.zeros(n, bool)
    rng = np.random.default_rng([seed, _S_PERM])
    tables, pool = _assign_blocks(rng, lens, block_size, shared, shared_prefix_blocks, pool)
    return Workload(
        name=name,
        seed=seed,
        num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        block_size=block_size,
        q_dtype=q_dtype,
        src_dtype=src_dtype,
        kv_dtype=kv_dtype,
        context_lens=lens,
        q_lens=qlens,
        block_tables=tables,
        num_blocks=pool,
        shared_seqs=shared,
        shared_prefix_blocks=shared_prefix_blocks,
        partition_size=partition_size,
        causal=causal,
    )


def make_config(idx: int, replica: int = 0) -> Workload:
    """The five named workloads.  ``replica`` > 0 draws an independent batch of
    the same shape (used to rotate pools so that timed steps do not re-read a
    batch that is still cached)."""
    seed = 2510 + idx + 7919 * replica
    rl = np.random.default_rng([seed, _S_LENS])
    name = CONFIG_NAMES[idx]
    if idx == 1:
        return make_workload(
            [1, 17, 33, 100], num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
            q_dtype="f32", pool=32, seed=seed, name=name,
        )
    if idx == 2:
        lens = rl.integers(512, 2048 + 1, size=64)
        return make_workload(lens, num_q_heads=32, num_kv_heads=8, head_dim=128, q_dtype="bf16",
                             seed=seed, name=name)
    if idx == 3:
        lens = rl.integers(256, 4096 + 1, size=128)
        return make_workload(lens, num_q_heads=32, num_kv_heads=8, head_dim=128, q_dtype="bf16",
                             src_dtype="bf16", kv_dtype="e5m2", seed=seed, name=name)
    if idx == 4:
        return make_workload(np.full(8, 32768), num_q_heads=64, num_kv_heads=8, head_dim=128,
                             q_dtype="bf16", partition_size=512, seed=seed, name=name)
    if idx == 5:
        n_new = rl.integers(256, 1024 + 1, size=4)
        cached = rl.integers(0, 2048 + 1, size=4)
        dec = rl.integers(128, 4096 + 1, size=128)
        lens = np.concatenate([cached + n_new, dec])
        qlens = np.concatenate([n_new, np.ones(128, np.int64)])
        prefix_blocks = 8
        eligible = np.nonzero(lens - qlens >= prefix_blocks * 16)[0]
        rs = np.random.default_rng([seed, _S_SHARE])
        n_share = int(0.25 * len(lens))
        pick = rs.choice(eligible, size=n_share, replace=False)
        shared = np.zeros(len(lens), bool)
        shared[pick] = True
        return make_workload(lens, q_lens=qlens, num_q_heads=32, num_kv_heads=8, head_dim=128,
                             q_dtype="bf16", shared_seqs=shared, shared_prefix_blocks=prefix_blocks,
                             causal=True, seed=seed, name=name)
    if idx == 6:
        # speculative verification: every sequence of the Llama-3-8B decode batch checks 4 draft
        # tokens at once (causal among them, the context counting them)
        lens = rl.integers(512, 2048 + 1, size=64)
        return make_workload(lens, q_lens=np.full(64, 4), num_q_heads=32, num_kv_heads=8, head_dim=128,
                             q_dtype="bf16", causal=True, seed=seed, name=name)
    if idx == 7:
        # the E5M2 decode batch's shape over an INT8 pool (codes plus a scale per row)
        lens = rl.integers(256, 4096 + 1, size=128)
        return make_workload(lens, num_q_heads=32, num_kv_heads=8, head_dim=128, q_dtype="bf16",
                             src_dtype="bf16", kv_dtype="int8", seed=seed, name=name)
    if idx == 9:
        # the packed prefill + decode step of workload 5 over an E5M2 pool
        import dataclasses

        base = make_config(5, replica)
        return dataclasses.replace(base, src_dtype="bf16", kv_dtype="e5m2", name=name)
    if idx == 8:
        # the same batch over a scaled FP8 E4M3 pool
        lens = rl.integers(256, 4096 + 1, size=128)
        return make_workload(lens, num_q_heads=32, num_kv_heads=8, head_dim=128, q_dtype="bf16",
                             src_dtype="bf16", kv_dtype="e4m3", seed=seed, name=name)
    raise ValueError(f"no workload {idx}")


def _shared_prefix_kv(w: Workload):
    rng = np.random.default_rng([w.seed, _S_SHARED_KV])
    shape = (w.shared_prefix_blocks * w.block_size, w.num_kv_heads, w.head_dim)
    return _normal(rng, shape, w.src_dtype), _normal(rng, shape, w.src_dtype)


def seq_kv(w: Workload, s: int, _shared=None):
    """Keys and values of every context position of sequence s, raw src dtype,
    each [L_s, Hkv, D]."""
    L = int(w.context_lens[s])
    rng = np.random.default_rng([w.seed, _S_KV, s])
    shape = (L, w.num_kv_heads, w.head_dim)
    k = _normal(rng, shape, w.src_dtype)
    v = _normal(rng, shape, w.src_dtype)
    if w.shared_seqs[s]:
        sk, sv = _shared if _shared is not None else _shared_prefix_kv(w)
        p = min(L, sk.shape[0])
        k[:p] = sk[:p]
        v[:p] = sv[:p]
    return k, v


def queries(w: Workload) -> np.ndarray:
    """Query rows packed without padding: [total_q, Hq, D] raw q dtype."""
    rng = np.random.default_rng([w.seed, _S_Q])
    return _normal(rng, (w.total_q, w.num_q_heads, w.head_dim), w.q_dtype)


def write_plan(w: Workload, phase: str = "all", seqs=None) -> WritePlan:
    """Rows for a cache write.

    phase 'all'    : every context position (a common prefix written once)
    phase 'cached' : positions before the query tokens (a varlen step's history)
    phase 'new'    : the query tokens' own positions (the step's write)
    """
    lens = w.context_lens.astype(np.int64)
    starts = np.zeros_like(lens)
    prefix = w.shared_prefix_blocks * w.block_size
    first = None
    for s in range(w.num_seqs):
        if w.shared_seqs[s]:
            if first is None:
                first = s
            else:
                starts[s] = prefix
    if phase == "all":
        ends = lens.copy()
    elif phase == "cached":
        ends = lens - w.q_lens
        starts = np.minimum(starts, ends)
    elif phase == "new":
        ends = lens.copy()
        starts = np.maximum(lens - w.q_lens, 0)
    else:
        raise ValueError(phase)
    sel = range(w.num_seqs) if seqs is None else seqs
    counts = np.zeros(w.num_seqs, np.int32)
    ks, vs = [], []
    shared = _shared_prefix_kv(w) if w.shared_prefix_blocks else None
    for s in sel:
        if ends[s] <= starts[s]:
            continue
        k, v = seq_kv(w, s, shared)
        ks.append(k[starts[s] : ends[s]])
        vs.append(v[starts[s] : ends[s]])
        counts[s] = ends[s] - starts[s]
    st = STORAGE[w.src_dtype]
    shape = (0, w.num_kv_heads, w.head_dim)
    k = np.concatenate(ks) if ks else np.zeros(shape, st)
    v = np.concatenate(vs) if vs else np.zeros(shape, st)
    return WritePlan(counts=counts, end_pos=ends.astype(np.int32), k=k, v=v)
