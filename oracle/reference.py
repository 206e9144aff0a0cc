"""Float64 CPU oracle for PagedAttention over a blocked KV cache.

TEST INFRASTRUCTURE ONLY (tests/, the smoke check, bench.py's cpu_baseline).

Sources, cited by page title and section:
  [CI]  Colossal-Inference release post ("AI大模型推理速度翻倍，Colossal-Inference开源发布"):
        sections "分块式KV缓存 (BlockedKeyValueCache)", "KV缓存量化 (KVCache Quant)",
        "分页注意力算法 (PagedAttention)", "连续批量化算法 (Continuous Batching)".
  [OPT] LLM inference optimisation overview ("AI 大模型推理优化技术详解"):
        sections "2.1.2 Paged Attention", "2.2.1 Flash Attention", "2.2.2 GQA",
        "2.6 低比特量化".
  [FW]  LLM inference frameworks page (LMDeploy section: KV Cache INT8 quantisation).

What the pages fix, restated:
  * Each sequence's keys and values are cut into blocks of a fixed number of
    tokens; consecutive logical blocks map through a block table to physical
    blocks that need not be contiguous [CI BlockedKeyValueCache; OPT 2.1.2].
    Where a block lives changes nothing in the result, so the oracle gathers
    the blocks back into contiguous arrays and runs textbook attention.
  * Query heads fall into groups that share one key/value head [OPT 2.2.2].
    Query head h reads KV head h // (Hq / Hkv)  (contiguous grouping).
  * The fp8 KV cache stores E5M2: the writer casts on store and the reader
    casts back to a wider type for the math [CI KVCache Quant].
  * Softmax can be reduced without the whole input at once (the running
    max/sum identity) [OPT 2.2.1]; ``attend_partitioned`` and
    ``combine_partials`` state that identity for split-KV.
  * Prefill and decode tokens are processed together as one packed 1-D token
    stream without padding [CI Continuous Batching]; ``paged_varlen``.
  * Low-bit KV caches save memory and traffic in a memory-bound step [OPT 2.6];
    an INT8 KV cache is one such format [FW: frameworks page, LMDeploy: KV Cache
    INT8].  No page fixes a scheme, so ``quantize_int8`` states the library's:
    symmetric, one float32 scale per (token, KV head) row.  ``quantize_e4m3`` is the same
    per-row scaling onto the FP8 E4M3 format's range (the "scaled FP8" variant).

Storage conventions: raw bits as in device memory -- f32 as float32, bf16 as
uint16 patterns, e5m2 as uint8 codes.  The oracle's own pool layout is
[num_blocks, block_size, num_kv_heads, head_dim]; it is independent of the
layout the library uses.
"""
from __future__ import annotations

import numpy as np

_STORAGE = {"f32": np.float32, "bf16": np.uint16, "e5m2": np.uint8}


# --------------------------------------------------------------------------
# exact decoding of stored values
# --------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32: widen exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to NaN
        return b.view(np.float32).astype(np.float64)


def e5m2_to_f64(codes) -> np.ndarray:
    """Value of an E5M2 code (1 sign, 5 exponent bits with bias 15, 2 mantissa
    bits; exponent 0 is subnormal, exponent 31 holds inf (mantissa 0) and NaN)
    [CI KVCache Quant names the format]."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 2) & 31
    m = c & 3
    sign = np.where(s == 1, -1.0, 1.0)
    val = np.where(e == 0, (m / 4.0) * 2.0**-14, (1.0 + m / 4.0) * np.exp2(e - 15.0))
    val = np.where(e == 31, np.where(m == 0, np.inf, np.nan), val)
    return sign * val


# Finite non-negative E5M2 magnitudes in code order 0x00..0x7B (ascending), then
# 2^16 standing where the next binade would start: code 0x7C (inf).
_E5M2_LADDER = np.append(e5m2_to_f64(np.arange(0x7C, dtype=np.uint8)), 65536.0)


def f64_to_e5m2(x) -> np.ndarray:
    """Round to the nearest E5M2 value, ties to the even code, overflow to inf.

    The pages say only that the writer casts to E5M2 [CI KVCache Quant]; the
    rounding is taken as IEEE round-to-nearest-even without saturation: a
    magnitude beyond the largest finite value (57344) goes to the nearest of
    {57344, 2^16 = inf}, the tie at 61440 going to the even code 0x7C (inf).
    NaN keeps its sign with code 0x7F.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    sign = (np.signbit(x).astype(np.uint8) << np.uint8(7)).astype(np.uint8)
    hi = np.clip(np.searchsorted(_E5M2_LADDER, a, side="left"), 0, 0x7C)
    lo = np.clip(hi - 1, 0, 0x7C)
    d_lo = a - _E5M2_LADDER[lo]
    d_hi = _E5M2_LADDER[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    code = np.where(a >= 65536.0, 0x7C, code)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8) | sign


def decode_storage(raw, dtype: str) -> np.ndarray:
    if dtype == "f64":  # values already decoded (e.g. a dequantised int8 pool)
        return np.asarray(raw, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(raw)
    if dtype == "e5m2":
        return e5m2_to_f64(raw)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# int8 rows with a scale  [OPT 2.6; FW LMDeploy KV Cache INT8; the scheme is this library's]
# --------------------------------------------------------------------------
def quantize_int8(x) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric int8 codes of every row (last axis) and one float32 scale per row.

    All in float32 arithmetic (IEEE, round to nearest even), which fixes every
    code bit for bit:
        amax  = max |x|            (maxNum: a NaN element is ignored)
        inv   = 127 / amax
        code  = clamp(rint(x * inv), -127, 127)   (clamp by minNum/maxNum: NaN -> -127)
        scale = amax / 127
    A row of zeros has codes 0 and scale 0.  The dequantised value is code * scale.
    """
    x32 = np.asarray(x, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        amax = np.fmax.reduce(np.abs(x32), axis=-1)
        inv = np.where(amax > 0, np.float32(127) / amax, np.float32(0)).astype(np.float32)
        prod = (x32 * inv[..., None]).astype(np.float32)
        code = np.fmin(np.fmax(np.rint(prod), np.float32(-127)), np.float32(127))
        scale = (amax / np.float32(127)).astype(np.float32)
    return code.astype(np.int8), scale


def dequantize_int8(codes, scales) -> np.ndarray:
    """code * scale in float64 (exact: an 8-bit integer times a float32)."""
    return np.asarray(codes, np.float64) * np.asarray(scales, np.float64)[..., None]


# --------------------------------------------------------------------------
# FP8 E4M3 rows with a scale  [OPT 2.6; the scheme is this library's]
# --------------------------------------------------------------------------
def e4m3_to_f64(codes) -> np.ndarray:
    """Value of an E4M3 code (OCP "FN" variant: 1 sign, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent 0 is subnormal, no infinities, S.1111.111 is NaN, largest finite 448)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    sign = np.where(s == 1, -1.0, 1.0)
    val = np.where(e == 0, (m / 8.0) * 2.0**-6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


# Finite non-negative E4M3 magnitudes in code order 0x00..0x7E (ascending).
_E4M3_LADDER = e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))


def f64_to_e4m3(x) -> np.ndarray:
    """Round to the nearest E4M3 value, ties to the even code, saturating: a magnitude at or
    above the largest finite value (448) gives 448.  NaN gives 0x7F (sign dropped)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    sign = (np.signbit(x).astype(np.uint8) << np.uint8(7)).astype(np.uint8)
    hi = np.clip(np.searchsorted(_E4M3_LADDER, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - _E4M3_LADDER[lo]
    d_hi = _E4M3_LADDER[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    code = np.where(a >= 448.0, 0x7E, code).astype(np.uint8) | sign
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def quantize_e4m3(x) -> tuple[np.ndarray, np.ndarray]:
    """E4M3 codes of every row (last axis) scaled to the format's range, and one float32 scale
    per row.  In float32 arithmetic (IEEE, round to nearest even):
        amax  = max |x|            (maxNum: a NaN element is ignored)
        inv   = 448 / amax         (0 when amax is 0 or NaN)
        code  = f64_to_e4m3(x * inv)   (the float32 product, rounded to E4M3 exactly once)
        scale = amax / 448
    The dequantised value is e4m3_to_f64(code) * scale."""
    x32 = np.asarray(x, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        amax = np.fmax.reduce(np.abs(x32), axis=-1)
        inv = np.where(amax > 0, np.float32(448) / amax, np.float32(0)).astype(np.float32)
        prod = (x32 * inv[..., None]).astype(np.float32)
        scale = (amax / np.float32(448)).astype(np.float32)
    return f64_to_e4m3(prod.astype(np.float64)), scale


def dequantize_e4m3(codes, scales) -> np.ndarray:
    """E4M3 value * scale in float64 (exact)."""
    return e4m3_to_f64(codes) * np.asarray(scales, np.float64)[..., None]


# --------------------------------------------------------------------------
# slot mapping and cache write  [CI BlockedKeyValueCache; CI KVCache Quant]
# --------------------------------------------------------------------------
def slot_mapping(block_tables, counts, end_pos, block_size: int) -> np.ndarray:
    """Slot of every written row.

    Sequence s writes ``counts[s]`` rows at logical positions
    end_pos[s]-counts[s] .. end_pos[s]-1; position p sits in logical block
    p // block_size at offset p % block_size, and the block table turns the
    logical block into a physical one: slot = table[p // B] * B + p % B.
    """
    bt = np.asarray(block_tables)
    out = []
    for s in range(len(counts)):
        n = int(counts[s])
        if n == 0:
            continue
        p = np.arange(int(end_pos[s]) - n, int(end_pos[s]), dtype=np.int64)
        out.append(bt[s, p // block_size].astype(np.int64) * block_size + p % block_size)
    if not out:
        return np.zeros(0, np.int32)
    return np.concatenate(out).astype(np.int32)


def new_pool(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int, dtype: str,
             fill_bits: int) -> np.ndarray:
    """Oracle pool [num_blocks, block_size, Hkv, D] of raw storage, every element
    set to ``fill_bits``."""
    st = _STORAGE[dtype]
    ut = {np.float32: np.uint32, np.uint16: np.uint16, np.uint8: np.uint8}[st]
    pool = np.full((num_blocks, block_size, num_kv_heads, head_dim), fill_bits, dtype=ut)
    return pool.view(st)


def _convert_rows(rows, src_dtype: str, cache_dtype: str) -> np.ndarray:
    if src_dtype == cache_dtype:
        return np.asarray(rows, dtype=_STORAGE[src_dtype])
    if cache_dtype == "e5m2" and src_dtype in ("bf16", "f32"):
        return f64_to_e5m2(decode_storage(rows, src_dtype))
    raise ValueError(f"no cast {src_dtype} -> {cache_dtype}")


def cache_write(pool, rows, slots, src_dtype: str, cache_dtype: str, block_size: int):
    """Store row r at (slots[r] // B, slots[r] % B); a negative slot skips the
    row.  With cache dtype e5m2 the row is cast on store [CI KVCache Quant]."""
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    conv = _convert_rows(np.asarray(rows)[keep], src_dtype, cache_dtype)
    pool[slots[keep] // block_size, slots[keep] % block_size] = conv
    return pool


def gather_kv(pool, table_row, context_len: int, block_size: int) -> np.ndarray:
    """Contiguous raw [L, Hkv, D] of one sequence: token t comes from physical
    block table_row[t // B], offset t % B.  Table entries past the last
    needed block are never read."""
    t = np.arange(int(context_len), dtype=np.int64)
    return pool[np.asarray(table_row, dtype=np.int64)[t // block_size], t % block_size]


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------
def attend(q, k, v, scale: float, q_pos=None) -> np.ndarray:
    """Textbook softmax attention in float64.

    q [nq, Hq, D], k/v [L, Hkv, D].  Query i sees keys 0..q_pos[i] (all L
    keys when q_pos is None).  Query head h uses KV head h // (Hq/Hkv)
    [OPT 2.2.2].  S = scale * q.k, w = exp(S - max S), o = sum(w v) / sum(w).
    An empty context gives a zero row.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    nq, hq, d = q.shape
    L, hkv, _ = k.shape
    out = np.zeros((nq, hq, d), np.float64)
    if L == 0 or nq == 0:
        return out
    g = hq // hkv
    pos = np.full(nq, L - 1, np.int64) if q_pos is None else np.asarray(q_pos, np.int64)
    visible = np.arange(L)[None, :] <= pos[:, None]
    for h in range(hq):
        kh = k[:, h // g, :]
        vh = v[:, h // g, :]
        s = scale * (q[:, h, :] @ kh.T)
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        w = np.where(visible, np.exp(s - m), 0.0)
        out[:, h, :] = (w @ vh) / w.sum(axis=1, keepdims=True)
    return out


def attend_partitioned(q, k, v, scale: float, partition: int, q_pos=None):
    """Per-partition softmax state of ``attend``: for tokens
    [j*P, (j+1)*P) of the context, m_j = max S, l_j = sum exp(S - m_j) and the
    normalised o_j = sum exp(S - m_j) v / l_j.  Returns (m [J,nq,Hq],
    l [J,nq,Hq], o [J,nq,Hq,D]); a partition a query cannot see has m = -inf,
    l = 0, o = 0."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    nq, hq, d = q.shape
    L, hkv, _ = k.shape
    g = hq // hkv
    pos = np.full(nq, L - 1, np.int64) if q_pos is None else np.asarray(q_pos, np.int64)
    nparts = max(-(-L // partition), 0)
    m = np.full((nparts, nq, hq), -np.inf)
    l = np.zeros((nparts, nq, hq))
    o = np.zeros((nparts, nq, hq, d))
    for j in range(nparts):
        lo, hi = j * partition, min((j + 1) * partition, L)
        tok = np.arange(lo, hi)
        visible = tok[None, :] <= pos[:, None]
        for h in range(hq):
            s = scale * (q[:, h, :] @ k[lo:hi, h // g, :].T)
            s = np.where(visible, s, -np.inf)
            mj = s.max(axis=1)
            seen = np.isfinite(mj)
            w = np.where(visible, np.exp(s - np.where(seen, mj, 0.0)[:, None]), 0.0)
            lj = w.sum(axis=1)
            m[j, :, h] = mj
            l[j, :, h] = lj
            o[j, :, h, :] = np.where(seen[:, None], (w @ v[lo:hi, h // g, :]) / np.where(seen, lj, 1.0)[:, None], 0.0)
    return m, l, o


def combine_partials(m, l, o) -> np.ndarray:
    """Merge partition states: M = max_j m_j, weight_j = exp(m_j - M) l_j,
    result = sum_j weight_j o_j / sum_j weight_j  [OPT 2.2.1, softmax reduced
    without the whole input]."""
    m = np.asarray(m, np.float64)
    l = np.asarray(l, np.float64)
    o = np.asarray(o, np.float64)
    big = m.max(axis=0)
    safe = np.where(np.isfinite(big), big, 0.0)
    wgt = np.where(np.isfinite(m), np.exp(m - safe[None]), 0.0) * l
    den = wgt.sum(axis=0)
    num = (wgt[..., None] * o).sum(axis=0)
    return np.where(den[..., None] > 0, num / np.where(den > 0, den, 1.0)[..., None], 0.0)


# --------------------------------------------------------------------------
# paged entry points, oracle side
# --------------------------------------------------------------------------
def paged_decode(pool_k, pool_v, kv_dtype: str, q_raw, q_dtype: str, block_tables, context_lens,
                 block_size: int, scale: float, seqs=None) -> np.ndarray:
    """Single-token decode over the blocked cache [CI PagedAttention]: query
    row s attends all context_lens[s] tokens of sequence s, read through its
    block table.  Returns float64 [len(seqs), Hq, D]."""
    q = decode_storage(q_raw, q_dtype)
    sel = range(q.shape[0]) if seqs is None else list(seqs)
    out = np.zeros((len(sel), q.shape[1], q.shape[2]))
    for i, s in enumerate(sel):
        L = int(context_lens[s])
        kk = decode_storage(gather_kv(pool_k, block_tables[s], L, block_size), kv_dtype)
        vv = decode_storage(gather_kv(pool_v, block_tables[s], L, block_size), kv_dtype)
        out[i] = attend(q[s : s + 1], kk, vv, scale)[0]
    return out


def paged_varlen(pool_k, pool_v, kv_dtype: str, q_raw, q_dtype: str, cu_seqlens_q, block_tables,
                 context_lens, block_size: int, scale: float, causal: bool = True,
                 seqs=None) -> dict:
    """Packed, unpadded mix of prefill chunks and decode tokens
    [CI Continuous Batching].  Sequence s owns query rows
    cu[s]..cu[s+1]-1, the last n_s = cu[s+1]-cu[s] tokens of its context of
    L_s tokens.  With ``causal`` query i of the sequence sees keys
    0..L_s-n_s+i (the mask aligned to the end of the context); otherwise all
    L_s keys.  Returns {s: float64 [n_s, Hq, D]}."""
    q = decode_storage(q_raw, q_dtype)
    cu = np.asarray(cu_seqlens_q, np.int64)
    sel = range(len(cu) - 1) if seqs is None else list(seqs)
    res = {}
    for s in sel:
        n = int(cu[s + 1] - cu[s])
        L = int(context_lens[s])
        kk = decode_storage(gather_kv(pool_k, block_tables[s], L, block_size), kv_dtype)
        vv = decode_storage(gather_kv(pool_v, block_tables[s], L, block_size), kv_dtype)
        pos = (L - n + np.arange(n)) if causal else None
        res[s] = attend(q[cu[s] : cu[s + 1]], kk, vv, scale, pos)
    return res
