"""Scaled 8-bit KV caches (INT8 and FP8 E4M3 codes with a float32 scale per row) on the GPU
against the float64 oracle (needs an MI355X).

Bars: the cache write's codes and scales bit-exact against oracle.quantize_int8 /
oracle.quantize_e4m3 on the same bf16 rows (a NaN scale where the oracle's is NaN), slots it
must not touch left as they were; block copies bit-exact; decode attention within the bf16 bar
of the oracle run on the dequantised pool (code value times scale in float64) at edge lengths,
every GQA group size, both head dims, whole and split contexts, and on sampled sequences of the
Llama-3-8B decode batch over each pool type at full size.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_251_amd as pa
from gpu_harness import (DEV, QUANT, SCALED, DeviceBatch, assert_close, oracle_int8_pools, scaled_canonical,
                         out_f64, poisoned_pool, to_device)
from workloads import make_config, make_workload, queries

pytestmark = pytest.mark.gpu


def _bf16_raw(x):
    """bf16 bit patterns of float32 values (round to nearest even, by torch on the host)."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _special_rows(D, rng):
    """Rows [n, D] (bf16 patterns) that reach every branch of the quantiser."""
    rows = []
    rows.append(_bf16_raw(np.zeros(D)))                                   # amax 0: codes 0, scale 0
    r = rng.standard_normal(D); r[3] = np.nan; rows.append(_bf16_raw(r))  # a NaN element is ignored
    rows.append(_bf16_raw(np.full(D, np.nan)))                            # all NaN: scale NaN, codes -127
    r = rng.standard_normal(D); r[5] = np.inf; rows.append(_bf16_raw(r))  # amax inf: inv 0
    r = rng.standard_normal(D); r[7] = -np.inf; rows.append(_bf16_raw(r))
    rows.append(_bf16_raw(rng.standard_normal(D) * 1e-39))                # subnormal: 127 / amax overflows
    rows.append(_bf16_raw(rng.standard_normal(D) * 3e37))                 # near the top of the range
    ties = np.concatenate([[127.0], np.arange(-63.5, 64.0, 1.0)])[:D]     # inv = 1: x.5 ties to even
    rows.append(_bf16_raw(ties))
    rows.append(_bf16_raw(np.concatenate([[254.0], 2 * np.arange(-32, 32) + 1.0, np.zeros(D)])[:D]))  # inv 0.5
    raw = _bf16_raw(rng.standard_normal(D))
    raw[0], raw[9] = 0x7F81, 0xFFC1  # signalling and negative NaN patterns
    rows.append(raw)
    rows.append(_bf16_raw(-np.abs(rng.standard_normal(D)) * 3))           # all negative
    return np.stack(rows)


KINDS = ["int8", "e4m3"]
WORKLOAD = {"int8": 7, "e4m3": 8}


def _raw_codes(c):
    return np.asarray(c).view(np.uint8)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("D,hkv", [(128, 3), (64, 2)])
def test_scaled_cache_write_bit_exact(kind, D, hkv):
    rng = np.random.default_rng(zlib.crc32(f"i8w{D}".encode()))
    special = _special_rows(D, rng)
    n_rand = 300
    scale = 10.0 ** rng.uniform(-6, 6, size=(n_rand, 1))
    rand = _bf16_raw(rng.standard_normal((n_rand, D)) * scale)
    rows_k = np.concatenate([special, rand])
    rows_v = np.concatenate([rand[::-1], special])
    T = rows_k.shape[0]
    # [T, Hkv, D]: head h of token t is row (t + 7h) mod T
    idx = (np.arange(T)[:, None] + 7 * np.arange(hkv)[None, :]) % T
    k, v = rows_k[idx], rows_v[idx]
    nb = (T + 15) // 16 + 3
    w = make_workload([16], num_q_heads=hkv, num_kv_heads=hkv, head_dim=D, q_dtype="bf16", kv_dtype=kind,
                      pool=nb)
    pk, pv = poisoned_pool(w, which="k"), poisoned_pool(w, which="v")
    before = scaled_canonical(pk.clone(), pv.clone())
    slots = rng.permutation(nb * 16)[:T].astype(np.int32)
    slots[[4, 40]] = [-1, nb * 16 + 3]  # skipped rows
    pa.kv_cache_write(to_device(k, "bf16"), to_device(v, "bf16"), pk, pv, torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    got = scaled_canonical(pk, pv)
    for name, src in (("k", k), ("v", v)):
        codes, scales = got[name]
        want_c, want_s = QUANT[kind][0](oracle.decode_storage(src, "bf16").astype(np.float32))
        want_c = _raw_codes(want_c)
        keep = slots >= 0
        keep &= slots < nb * 16
        blk, off = slots[keep] // 16, slots[keep] % 16
        got_c, got_s = codes[blk, off], scales[blk, off]
        bad = np.nonzero(got_c != want_c[keep])
        assert bad[0].size == 0, f"{name}: codes differ at {list(zip(*bad))[:5]}"
        nan_w = np.isnan(want_s[keep])
        assert np.array_equal(np.isnan(got_s), nan_w), name
        assert np.array_equal(got_s[~nan_w].view(np.uint32), want_s[keep][~nan_w].view(np.uint32)), name
        # every slot not written keeps the poison (codes and scale)
        written = np.zeros((nb, 16), bool)
        written[blk, off] = True
        pc, ps = before[name]
        assert np.array_equal(codes[~written], pc[~written]), name
        assert np.all(np.isnan(scales[~written])), name


@pytest.mark.parametrize("kind", KINDS)
def test_scaled_copy_blocks_bit_exact(kind):
    rng = np.random.default_rng(5)
    nb, hkv, D = 24, 2, 128
    # a key block holds the codes and both rows' scales, a value block the codes only
    kc = torch.from_numpy(rng.integers(-128, 128, size=(nb, hkv, 16 * D + 128), dtype=np.int8)).to(DEV)
    vc = torch.from_numpy(rng.integers(-128, 128, size=(nb, hkv, 16, D), dtype=np.int8)).to(DEV)
    pairs = np.array([[1, 20], [2, 21], [3, 3], [-1, 5], [7, 22]], np.int32)
    kx, vx = kc.cpu().clone(), vc.cpu().clone()
    for s, d in pairs:
        if 0 <= s < nb and 0 <= d < nb and s != d:
            kx[d], vx[d] = kx[s], vx[s]
    pa.copy_blocks(kc.view(SCALED[kind]), vc.view(SCALED[kind]), torch.from_numpy(pairs).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(kc.cpu(), kx) and torch.equal(vc.cpu(), vx)


EDGE_LENS = [0, 1, 2, 15, 16, 17, 255, 256, 257, 511, 512, 513, 1000]


def _check_pools_match(b, w, o, seqs=None):
    """The GPU-written pools hold exactly the oracle's codes and scales on every slot written."""
    got = scaled_canonical(b.pk, b.pv)
    for name in ("k", "v"):
        codes, scales = got[name]
        oc, os_, oset, _ = o[name]
        assert np.array_equal(codes[oset], oc[oset]), name
        assert np.array_equal(scales[oset].view(np.uint32), os_[oset].view(np.uint32)), name


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("D,hkv,G", [
    (128, 2, 1), (128, 2, 2), (128, 1, 4), (128, 1, 8), (128, 1, 16), (64, 2, 4), (64, 1, 8), (64, 1, 16),
])
def test_scaled_decode_edge_lengths_gqa_and_head_dims(kind, D, hkv, G):
    w = make_workload(EDGE_LENS, num_q_heads=hkv * G, num_kv_heads=hkv, head_dim=D, q_dtype="bf16",
                      src_dtype="bf16", kv_dtype=kind, seed=zlib.crc32(f"i8{D}{hkv}{G}".encode()) % 1000)
    b = DeviceBatch(w)
    o = oracle_int8_pools(w)
    _check_pools_match(b, w, o)
    ref = oracle.paged_decode(o["k"][3], o["v"][3], "f64", queries(w), "bf16", w.block_tables, w.context_lens,
                              16, w.scale)
    for part in (0, 256, 512, -1):
        got = out_f64(b.decode(part), "bf16")
        err = assert_close(got, ref, "bf16", f"{kind} D{D} G{G} partition {part}")
        assert np.all(got[0] == 0.0)  # empty context
    print(f"{kind} D{D} G{G}: max abs err {err:.2e}")


@pytest.mark.parametrize("kind", KINDS)
def test_scaled_decode_large_values(kind):
    """Rows with large magnitudes (value scales up to ~2^7, probabilities up to 2^8 before the
    lazy max moves): the f16 product of probability and value scale stays in range."""
    w = make_workload([700, 33], num_q_heads=8, num_kv_heads=2, head_dim=128, q_dtype="bf16", src_dtype="bf16",
                      kv_dtype=kind, seed=77)
    b = DeviceBatch(w, phases=())
    from workloads import write_plan

    plan = write_plan(w, "all")
    big_k = _bf16_raw(oracle.decode_storage(plan.k, "bf16") * 4.0)
    big_v = _bf16_raw(oracle.decode_storage(plan.v, "bf16") * 3000.0)
    cu = torch.from_numpy(plan.cu).to(DEV)
    end = torch.from_numpy(plan.end_pos).to(DEV)
    slots = pa.slot_mapping(cu, end, b.tables, plan.num_tokens, w.num_blocks, 16)
    pa.kv_cache_write(to_device(big_k, "bf16"), to_device(big_v, "bf16"), b.pk, b.pv, slots)
    quant, dequant = QUANT[kind]
    ck, sk = quant(oracle.decode_storage(big_k, "bf16").astype(np.float32))
    cv, sv = quant(oracle.decode_storage(big_v, "bf16").astype(np.float32))
    kd, vd = dequant(ck, sk), dequant(cv, sv)
    q = oracle.decode_storage(queries(w), "bf16")
    ref, start = [], 0
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        ref.append(oracle.attend(q[s : s + 1], kd[start : start + L], vd[start : start + L], w.scale)[0])
        start += L
    ref = np.stack(ref)
    for part in (0, 256):
        got = out_f64(b.decode(part), "bf16")
        # the bar scales with the values: 1e-2 of the value range's unit (3000 here)
        assert np.all(np.isfinite(got))
        diff = np.abs(got - ref)
        bound = 3000.0 * 1e-2 + 2.0**-8 * np.abs(ref)
        assert (diff <= bound).all(), f"partition {part}: {diff.max():.3e}"


def _sample(w, k, seed):
    rng = np.random.default_rng(seed)
    order = np.argsort(w.context_lens)
    pick = set([int(order[0]), int(order[-1])]) | set(rng.choice(w.num_seqs, size=k, replace=False).tolist())
    return sorted(pick)


@pytest.mark.parametrize("kind", KINDS)
def test_scaled_decode_full_size_sampled(kind):
    w = make_config(WORKLOAD[kind])
    b = DeviceBatch(w)
    sel = _sample(w, 6, 41)
    o = oracle_int8_pools(w, seqs=sel)
    _check_pools_match(b, w, o)
    ref = oracle.paged_decode(o["k"][3], o["v"][3], "f64", queries(w), "bf16", w.block_tables, w.context_lens, 16,
                              w.scale, seqs=sel)
    for part in (-1, 512):
        out = out_f64(b.decode(part), "bf16")[sel]
        err = assert_close(out, ref, "bf16", f"{kind} full size partition {part}")
        print(f"{kind} full size partition {part}: max abs err {err:.2e}")


# ---------------------------------------------------------------- fused append on scaled pools
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("D,G", [(128, 4), (128, 8), (64, 4), (64, 16)])
def test_scaled_append_is_bit_identical_to_write_then_decode(kind, D, G):
    """paged_attention_decode_append quantises each sequence's newest K/V row in the kernel (INT8
    and FP8 E4M3 pools, with the cache write's rule): the pools it leaves and its output equal,
    byte for byte, the quantising kv_cache_write followed by the decode, and both match the
    oracle's codes, scales and attention."""
    from workloads import STORAGE, seq_kv

    w = make_workload([1, 2, 16, 17, 32, 33, 300, 513, 0], num_q_heads=2 * G, num_kv_heads=2, head_dim=D,
                      q_dtype="bf16", src_dtype="bf16", kv_dtype=kind,
                      seed=zlib.crc32(f"app{kind}{D}{G}".encode()) % 1000)
    o = oracle_int8_pools(w)
    ref = oracle.paged_decode(o["k"][3], o["v"][3], "f64", queries(w), "bf16", w.block_tables, w.context_lens,
                              16, w.scale)
    kn = np.zeros((w.num_seqs, w.num_kv_heads, w.head_dim), STORAGE["bf16"])
    vn = np.zeros_like(kn)
    for s in range(w.num_seqs):
        if w.context_lens[s] > 0:
            ks, vs = seq_kv(w, s)
            kn[s], vn[s] = ks[-1], vs[-1]
    k = to_device(kn, "bf16")
    v = to_device(vn, "bf16")
    for part in (0, 256):
        a = DeviceBatch(w, phases=("cached",))
        b = DeviceBatch(w, phases=("cached",))
        a.write("new")
        out_sep = a.decode(part)
        out_fused = pa.paged_attention_decode_append(b.q, k, v, b.pk, b.pv, b.tables, b.lens, w.max_context_len,
                                                     w.scale, partition_size=part)
        assert torch.equal(out_sep.view(torch.int16), out_fused.view(torch.int16)), f"{kind} partition {part}"
        assert torch.equal(a.pk.view(torch.uint8), b.pk.view(torch.uint8))
        assert torch.equal(a.pv.view(torch.uint8), b.pv.view(torch.uint8))
        _check_pools_match(b, w, o)
        assert_close(out_f64(out_fused, "bf16"), ref, "bf16", f"{kind} append D{D} G{G} partition {part}")
