"""A continuous-batching run driven by the step scheduler, on the GPU (needs an MI355X).

The host scheduler (pa_sched_*) and block manager decide every step; the library's kernels
carry it out: block copies, slot mapping, the cache write of the step's rows, and the packed
attention (paged_attention_varlen for prefill steps, paged_attention_decode for decode steps).
Keys, values and queries are functions of a token's whole prefix (as in a model), so a prefix
reused from the cache holds the right rows for every sequence.  Every query row of every step
is checked against the float64 oracle attending over that sequence's rows in position order.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_251_amd as pa
from gpu_harness import DEV, assert_close, out_f64, to_device

pytestmark = pytest.mark.gpu

HKV, G, D, B = 2, 4, 128, 16


def _bf16_raw(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _prefix_keys(tokens):
    h, keys = 0, []
    for t in tokens:
        h = zlib.crc32(np.int64([h, t]).tobytes())
        keys.append(h)
    return keys


def _rows(key, what, shape):
    rng = np.random.default_rng([key, what])
    return _bf16_raw(rng.standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("pool,ratio", [(48, 1.0), (20, 0.5)])
def test_scheduled_serving_run_matches_the_oracle(pool, ratio):
    rng = np.random.default_rng(pool)
    m = pa.BlockManager(pool, B)
    sched = pa.Scheduler(m, max_running=8, max_batch_tokens=320, prefill_ratio=ratio, max_blocks_per_seq=20)
    kc = torch.zeros((pool, HKV, B, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    known = {}  # request -> every token it knows (prompt + produced)
    system = [int(t) for t in rng.integers(0, 50, size=40)]  # a shared system prompt
    nid, checked, kinds, preempted = 0, 0, [0, 0, 0], 0
    scale = 1.0 / np.sqrt(D)
    for step in range(60):
        for _ in range(int(rng.poisson(0.7)) if nid < 24 else 0):
            body = [int(t) for t in rng.integers(0, 50, size=int(rng.integers(1, 60)))]
            prompt = (system if rng.random() < 0.6 else []) + body
            sched.add_request(nid, prompt, int(rng.integers(1, 30)))
            known[nid] = list(prompt)
            nid += 1
        s = sched.step()
        kinds[s["kind"]] += 1
        preempted += len(s["preempted"])
        n = len(s["seq_ids"])
        if n == 0:
            sched.commit([])
            continue
        if s["copies"]:
            pa.copy_blocks(kc, vc, torch.tensor(s["copies"], dtype=torch.int32, device=DEV))
        cu = s["cu_seqlens_q"]
        lens = s["context_lens"]
        # rows of this step: positions L - q .. L - 1 of each sequence
        k_rows, v_rows, q_rows = [], [], []
        for i, rid in enumerate(s["seq_ids"]):
            toks = known[int(rid)][: lens[i]]
            keys = _prefix_keys(toks)
            assert s["input_tokens"][cu[i]:cu[i + 1]].tolist() == toks[lens[i] - (cu[i + 1] - cu[i]):]
            for p in range(lens[i] - (cu[i + 1] - cu[i]), lens[i]):
                k_rows.append(_rows(keys[p], 1, (HKV, D)))
                v_rows.append(_rows(keys[p], 2, (HKV, D)))
                q_rows.append(_rows(keys[p], 3, (HKV * G, D)))
        cu_d = torch.from_numpy(cu).to(DEV)
        lens_d = torch.from_numpy(lens).to(DEV)
        tables = torch.from_numpy(s["block_tables"]).to(DEV)
        slots = pa.slot_mapping(cu_d, lens_d, tables, s["total_q"], pool, B)
        pa.kv_cache_write(to_device(np.stack(k_rows), "bf16"), to_device(np.stack(v_rows), "bf16"), kc, vc, slots)
        q = to_device(np.stack(q_rows), "bf16")
        if s["kind"] == 1:
            out = pa.paged_attention_varlen(q, kc, vc, cu_d, lens_d, tables, s["max_q_len"], s["max_context_len"], scale,
                                            causal=True)
        else:
            out = pa.paged_attention_decode(q, kc, vc, tables, lens_d, s["max_context_len"], scale)
        got = out_f64(out, "bf16")
        # oracle: each row attends positions 0 .. its own, rows regenerated from the tokens
        for i, rid in enumerate(s["seq_ids"]):
            toks = known[int(rid)][: lens[i]]
            keys = _prefix_keys(toks)
            kk = oracle.decode_storage(np.stack([_rows(h, 1, (HKV, D)) for h in keys]), "bf16")
            vv = oracle.decode_storage(np.stack([_rows(h, 2, (HKV, D)) for h in keys]), "bf16")
            first = lens[i] - (cu[i + 1] - cu[i])
            for r in range(cu[i], cu[i + 1]):
                p = first + (r - cu[i])
                qr = oracle.decode_storage(q_rows[r][None], "bf16")
                ref = oracle.attend(qr, kk[: p + 1], vv[: p + 1], scale)
                assert_close(got[r : r + 1], ref, "bf16", f"step {step} request {rid} position {p}")
                checked += 1
        nxt = [int(t) for t in rng.integers(0, 50, size=n)]
        for i, rid in enumerate(s["seq_ids"]):
            known[int(rid)].append(nxt[i])
        sched.commit(nxt, [bool(f) for f in rng.random(n) < 0.03])
    print(f"pool {pool}: {kinds[1]} prefill and {kinds[2]} decode steps, {preempted} preemptions, "
          f"{checked} rows checked, stats {sched.stats()}")
    assert kinds[1] > 0 and kinds[2] > 0 and checked > 100
    if pool == 20:
        assert preempted > 0
