"""GPU side of block management (needs an MI355X).

paged_kv_copy_blocks is compared byte for byte with the same copies done on the host; then the
host block manager drives a small serving run -- prompts that share prefixes, forks and appends
that copy a shared partial block -- through slot mapping, cache write, block copies and decode,
and every sequence's attention is checked against the float64 oracle on its logical rows.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_251_amd as pa
from gpu_harness import DEV, assert_close, out_f64, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,elem", [("bf16", torch.int16), ("e5m2", torch.uint8), ("f32", torch.int32)])
def test_copy_blocks_bit_exact(dtype, elem):
    rng = np.random.default_rng(zlib.crc32(dtype.encode()))
    nb, hkv, B, D = 40, 4, 16, 64
    info = torch.iinfo(elem)
    raw = rng.integers(info.min, info.max, size=(nb, hkv, B, D), endpoint=True)
    kc = torch.from_numpy(raw.astype(np.int64)).to(elem).to(DEV)
    vc = torch.from_numpy((raw[::-1].copy()).astype(np.int64)).to(elem).to(DEV)
    store = {"bf16": torch.bfloat16, "e5m2": torch.uint8, "f32": torch.float32}[dtype]
    srcs = rng.permutation(20)[:8]
    dsts = 20 + rng.permutation(20)[:8]
    pairs = np.stack([srcs, dsts], 1).astype(np.int32)
    pairs = np.concatenate([pairs, [[-1, 30], [3, 40], [5, 5]]]).astype(np.int32)  # skipped
    kx, vx = kc.cpu().clone(), vc.cpu().clone()
    for s, d in pairs:
        if 0 <= s < nb and 0 <= d < nb and s != d:
            kx[d], vx[d] = kx[s], vx[s]
    pa.copy_blocks(kc.view(store), vc.view(store), torch.from_numpy(pairs).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(kc.cpu(), kx) and torch.equal(vc.cpu(), vx)


def _bf16_raw(x):
    """bf16 bit patterns of float32 values (round to nearest even, by torch on the host)."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rows(prefix_key, hkv, D):
    """K/V rows of a token: a function of the whole prefix (as in a model), so equal prefixes
    give equal rows and shared blocks hold the right values for every sequence."""
    rng = np.random.default_rng(prefix_key)
    k = rng.standard_normal((hkv, D)).astype(np.float32)
    v = rng.standard_normal((hkv, D)).astype(np.float32)
    return k, v


def test_manager_driven_decode_with_sharing_forks_and_copy_on_write():
    rng = np.random.default_rng(11)
    B, nb, hkv, G, D = 16, 96, 2, 4, 128
    m = pa.BlockManager(nb, B)
    kc = torch.zeros((nb, hkv, B, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    seqs = {}  # id -> token list

    def prefix_keys(tokens):
        h, keys = 0, []
        for t in tokens:
            h = zlib.crc32(np.int64([h, t]).tobytes())
            keys.append(h)
        return keys

    def write(sid, first):
        """Write rows first .. end of sequence sid at the slots its table gives."""
        toks = seqs[sid]
        table, n = m.block_table(sid)
        keys = prefix_keys(toks)
        rows = [_rows(keys[p], hkv, D) for p in range(first, n)]
        if not rows:
            return
        k = np.stack([r[0] for r in rows]).astype(np.float32)
        v = np.stack([r[1] for r in rows]).astype(np.float32)
        slots = np.array([table[p // B] * B + p % B for p in range(first, n)], np.int32)
        kb = to_device(_bf16_raw(k), "bf16")
        vb = to_device(_bf16_raw(v), "bf16")
        pa.kv_cache_write(kb, vb, kc, vc, torch.from_numpy(slots).to(DEV))

    prompt = [int(t) for t in rng.integers(0, 100, size=70)]
    seqs[0] = prompt
    assert m.add_sequence(0, len(prompt), prompt) == 0
    write(0, 0)
    # a second prompt with the same first 48 tokens reuses 3 blocks
    seqs[1] = prompt[:48] + [int(t) for t in rng.integers(0, 100, size=13)]
    cached = m.add_sequence(1, len(seqs[1]), seqs[1])
    assert cached == 48
    write(1, cached)
    # a fork of sequence 0 and appends to both: the shared partial block is copied first
    m.fork(0, 2)
    seqs[2] = list(seqs[0])
    for sid in (2, 0, 1):
        new = [int(t) for t in rng.integers(0, 100, size=5)]
        n_before = len(seqs[sid])
        copies = m.append(sid, len(new), new)
        # the fork shares sequence 0's partly filled last block: the first append copies it
        assert bool(copies) == (sid == 2), (sid, copies)
        if copies:
            pa.copy_blocks(kc, vc, torch.tensor(copies, dtype=torch.int32, device=DEV))
        seqs[sid] = seqs[sid] + new
        write(sid, n_before)
    torch.cuda.synchronize()

    ids = sorted(seqs)
    tables = [m.block_table(s)[0] for s in ids]
    lens = np.array([len(seqs[s]) for s in ids], np.int32)
    mb = max(len(t) for t in tables)
    bt = np.full((len(ids), mb), -1, np.int32)
    for i, t in enumerate(tables):
        bt[i, : len(t)] = t
    q = rng.standard_normal((len(ids), hkv * G, D)).astype(np.float32)
    qb = to_device(_bf16_raw(q), "bf16")
    out = pa.paged_attention_decode(qb, kc, vc, torch.from_numpy(bt).to(DEV), torch.from_numpy(lens).to(DEV),
                                    int(lens.max()), 1.0 / np.sqrt(D), partition_size=0)
    got = out_f64(out, "bf16")
    qd = oracle.decode_storage(_bf16_raw(q), "bf16")
    for i, sid in enumerate(ids):
        keys = prefix_keys(seqs[sid])
        k = np.stack([_rows(h, hkv, D)[0] for h in keys])
        v = np.stack([_rows(h, hkv, D)[1] for h in keys])
        kd = oracle.decode_storage(_bf16_raw(k), "bf16")
        vd = oracle.decode_storage(_bf16_raw(v), "bf16")
        ref = oracle.attend(qd[i : i + 1], kd, vd, 1.0 / np.sqrt(D))
        assert_close(got[i : i + 1], ref, "bf16", f"sequence {sid}")
