#!/usr/bin/env python3
"""Paged decode attention benchmark on one MI355X.

One step = the whole decode path for one batch: slot mapping of each sequence's
newest token, the cache write of its K/V row (cast to E5M2 for an fp8 cache,
quantised with a per-row scale for an INT8 or E4M3 cache), the paged attention partition pass and, when contexts are split, the reduce
pass.  The timed step runs these as one fused launch
(paged_attention_decode_append; plus the reduce kernel when split); the same
step as three separate calls (slot mapping, kv_cache_write, decode) is timed
too and reported as ``unfused``.  Several independently seeded
batches of the same shape are resident and steps rotate over them, so a timed
step never re-reads a pool that an earlier step left in the 256 MB Infinity
Cache.  Inputs are synthetic (seeded N(0,1) values with the workload's shapes).

Prints one JSON line:
  value        = KV bytes the method must read per step / step time, GB/s
  roofline     = the partition kernel alone, timed with HIP events on its stream
  cpu_baseline = the float64 oracle on the host, on a bounded sample of the batch
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attn: KV-read HBM GB/s (% of peak) + seq-steps/sec, 1 GPU"
HBM_PEAK_GBS = 8000.0
KV_BYTES = {"f32": 4, "bf16": 2, "e5m2": 1, "int8": 1, "e4m3": 1}
SCALED = ("int8", "e4m3")  # pools with a float32 scale per (token, KV head) row


def launch_stats(ms) -> dict:
    """Median, min and 90th percentile of per-launch times (ms) in microseconds."""
    import numpy as np

    us = np.asarray(ms, dtype=np.float64) * 1e3
    return {"median_us": round(float(np.median(us)), 3), "min_us": round(float(us.min()), 3),
            "p90_us": round(float(np.percentile(us, 90)), 3), "launches": int(us.size)}


def row_bytes(w) -> int:
    """Pool bytes of one (token, KV head) row: head_dim elements, plus the float32 scale of an
    INT8 row."""
    return w.head_dim * KV_BYTES[w.kv_dtype] + (4 if w.kv_dtype in SCALED else 0)


LEAD_IN_CYCLES = 20_000_000


def resident_lens(batches) -> str:
    """Context-length range over every resident batch (the timed steps rotate over them)."""
    lo = min(int(b.w.context_lens.min()) for b in batches)
    hi = max(int(b.w.context_lens.max()) for b in batches)
    return f"{lo}..{hi}"


def lead_in(torch, stream) -> None:
    """Keep the GPU busy (a spin kernel, not timed) while the host queues the first steps, so the
    timed region opens on queued GPU work: what it measures is the device's time per step, not the
    host's latency in issuing the first launch."""
    with torch.cuda.stream(stream):
        torch.cuda._sleep(LEAD_IN_CYCLES)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, help="workload 1-9 (1-4 decode, 5 packed prefill + decode, 6 speculative verification of 4 tokens, "
                    "7 decode over an INT8 pool, 8 over a scaled FP8 E4M3 pool, 9 the packed step over an E5M2 "
                    "pool)")
    ap.add_argument("--replicas", type=int, default=0, help="resident batches to rotate (0: enough for >= 1.2 GB)")
    ap.add_argument("--partition", type=int, default=None, help="partition tokens (default: workload's, else auto)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic", type=str, default=os.path.join(ROOT, "profiles", "hbm_traffic.json"),
                    help="measured HBM bytes per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, calibrated)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only copy BYTES between two device buffers 3 times (calibrates HBM byte counters)")
    return ap.parse_args()


def copy_calibration(nbytes: int) -> None:
    """A plain device copy of known size: under rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE
    per dispatch against nbytes give the scale of the counters."""
    import torch

    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "dispatches": 3}), flush=True)


class Batch:
    """One resident batch: pools filled up to each sequence's previous token, and the
    arguments of every call of a step, prepared once."""

    def __init__(self, w, partition, pa, torch, to_dev):
        from workloads import POISON_BITS, queries, write_plan

        dev = "cuda:0"
        self.w = w
        self.tables = torch.from_numpy(w.block_tables).to(dev)
        self.lens = torch.from_numpy(w.context_lens).to(dev)
        if w.kv_dtype in SCALED:  # key pool: codes, key scales, value scales; value pool: codes; every word NaN
            kwords = (w.num_blocks, w.num_kv_heads, (w.block_size * w.head_dim + 128) // 4)
            vwords = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim // 4)
            store = torch.int8 if w.kv_dtype == "int8" else torch.float8_e4m3fn
            self.pk = torch.full(kwords, POISON_BITS[w.kv_dtype], dtype=torch.int32, device=dev).view(store)
            self.pv = torch.full(vwords, POISON_BITS[w.kv_dtype], dtype=torch.int32, device=dev).view(store)
        else:
            shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
            ints = {"f32": torch.int32, "bf16": torch.int16, "e5m2": torch.uint8}[w.kv_dtype]
            store = {"f32": torch.float32, "bf16": torch.bfloat16, "e5m2": torch.uint8}[w.kv_dtype]
            self.pk = torch.full(shape, POISON_BITS[w.kv_dtype], dtype=ints, device=dev).view(store)
            self.pv = self.pk.clone()
        # every pool kind takes the fused append (an INT8 or E4M3 pool's new row is quantised in the
        # kernel with the cache write's rule)
        self.fused = True
        hist = write_plan(w, "cached")
        slots = pa.slot_mapping(torch.from_numpy(hist.cu).to(dev), torch.from_numpy(hist.end_pos).to(dev),
                                self.tables, hist.num_tokens, w.num_blocks)
        pa.kv_cache_write(to_dev(hist.k, w.src_dtype), to_dev(hist.v, w.src_dtype), self.pk, self.pv, slots)
        new = write_plan(w, "new")
        self.cu = torch.from_numpy(new.cu).to(dev)
        self.end = torch.from_numpy(new.end_pos).to(dev)
        self.knew = to_dev(new.k, w.src_dtype)
        self.vnew = to_dev(new.v, w.src_dtype)
        self.ntok = new.num_tokens
        self.slots = torch.empty(self.ntok, dtype=torch.int32, device=dev)
        self.q = to_dev(queries(w), w.q_dtype)
        self.out = torch.empty_like(self.q)
        g = w.gqa_group
        self.partition = partition
        need = pa.workspace_size(w.num_seqs, w.num_kv_heads, g, w.head_dim, w.max_context_len, partition)
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        self.resolved = partition if partition >= 0 else pa.auto_partition(w.num_seqs, w.num_kv_heads, g, w.head_dim,
                                                                            w.max_context_len)
        self.split = need > 0
        qd = pa.binding.dtype_code(self.q)
        kd = pa.binding.dtype_code(self.pk)
        sd = pa.binding.dtype_code(self.knew)
        n, hkv, d, bs, nb = w.num_seqs, w.num_kv_heads, w.head_dim, w.block_size, w.num_blocks
        mb, ml = w.max_blocks_per_seq, w.max_context_len
        P = lambda t: t.data_ptr()
        self.args_slot = (P(self.slots), P(self.cu), P(self.end), P(self.tables), mb, n, self.ntok, bs, nb)
        self.args_write = (P(self.knew), P(self.vnew), P(self.pk), P(self.pv), P(self.slots), self.ntok, hkv, d, bs,
                           nb, sd, kd)
        self.args_parts = (P(self.out), P(self.q), P(self.pk), P(self.pv), P(self.tables), mb, P(self.lens), n, hkv, g,
                           d, bs, nb, ml, w.scale, qd, kd, partition, P(self.ws), self.ws.numel())
        self.args_reduce = (P(self.out), P(self.lens), mb, n, hkv, g, d, bs, ml, qd, kd, partition, P(self.ws),
                            self.ws.numel())
        self.args_append = (P(self.out), P(self.q), P(self.knew), P(self.vnew), P(self.pk), P(self.pv), P(self.tables),
                            mb, P(self.lens), n, hkv, g, d, bs, nb, ml, w.scale, qd, kd, partition,
                            pa.binding.PA_APPEND_SKIP_REDUCE, P(self.ws), self.ws.numel())
        self.kv_bytes = int(w.context_lens.astype("int64").sum()) * hkv * 2 * row_bytes(w)


class VarlenBatch:
    """One resident packed batch (prefill chunks first, then decode tokens): pools hold every
    sequence's history; a step writes the new tokens' K/V and attends."""

    def __init__(self, w, partition, pa, torch, to_dev):
        from workloads import POISON_BITS, queries, write_plan

        dev = "cuda:0"
        self.w = w
        self.tables = torch.from_numpy(w.block_tables).to(dev)
        self.lens = torch.from_numpy(w.context_lens).to(dev)
        shape = (w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim)
        if w.kv_dtype == "e5m2":
            self.pk = torch.full(shape, POISON_BITS["e5m2"], dtype=torch.uint8, device=dev)
        else:
            self.pk = torch.full(shape, POISON_BITS["bf16"], dtype=torch.int16, device=dev).view(torch.bfloat16)
        self.pv = self.pk.clone()
        hist = write_plan(w, "cached")
        slots = pa.slot_mapping(torch.from_numpy(hist.cu).to(dev), torch.from_numpy(hist.end_pos).to(dev),
                                self.tables, hist.num_tokens, w.num_blocks)
        pa.kv_cache_write(to_dev(hist.k, "bf16"), to_dev(hist.v, "bf16"), self.pk, self.pv, slots)
        new = write_plan(w, "new")
        self.cu_new = torch.from_numpy(new.cu).to(dev)
        self.end_new = torch.from_numpy(new.end_pos).to(dev)
        self.knew, self.vnew = to_dev(new.k, "bf16"), to_dev(new.v, "bf16")
        self.ntok = new.num_tokens
        self.slots = torch.empty(self.ntok, dtype=torch.int32, device=dev)
        self.q = to_dev(queries(w), "bf16")
        self.out = torch.empty_like(self.q)
        self.cu_q = torch.from_numpy(w.cu_seqlens_q).to(dev)
        n, hkv, g, d, bs, nb = w.num_seqs, w.num_kv_heads, w.gqa_group, w.head_dim, w.block_size, w.num_blocks
        mb, ml = w.max_blocks_per_seq, w.max_context_len
        n_pre = int((w.q_lens > 1).sum())  # prefill chunks are packed first
        # the full batch and the prefill-only / decode-only sub-batches may resolve differently
        need = max(pa.workspace_size(k, hkv, g, d, ml, partition) for k in (n, n_pre, n - n_pre) if k > 0)
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        self.resolved = partition if partition >= 0 else pa.auto_partition(n, hkv, g, d, ml)
        P = lambda t: t.data_ptr()
        bf = pa.binding.PA_BF16
        kd = pa.binding.dtype_code(self.pk)
        self.args_slot = (P(self.slots), P(self.cu_new), P(self.end_new), P(self.tables), mb, n, self.ntok, bs, nb)
        self.args_write = (P(self.knew), P(self.vnew), P(self.pk), P(self.pv), P(self.slots), self.ntok, hkv, d, bs,
                           nb, bf, kd)

        def varlen_args(s0, s1, part):
            rows0 = int(w.cu_seqlens_q[s0])
            cu = torch.from_numpy((w.cu_seqlens_q[s0 : s1 + 1] - rows0).astype("int32")).to(dev)
            self._keep.append(cu)
            qlen = int(w.q_lens[s0:s1].max())
            qoff = rows0 * w.num_q_heads * d * 2
            return (P(self.out) + qoff, P(self.q) + qoff, P(self.pk), P(self.pv), P(cu), P(self.lens) + 4 * s0,
                    P(self.tables) + 4 * mb * s0, mb, s1 - s0, int(w.q_lens[s0:s1].sum()), qlen, hkv, g, d, bs, nb,
                    ml, w.scale, 1, bf, kd, part, P(self.ws), self.ws.numel())

        self._keep = []
        self.args_varlen = varlen_args(0, n, partition)
        # the sub-batches run with the full batch's partition size, as its rows do in the full step
        self.args_prefill_only = varlen_args(0, n_pre, self.resolved) if n_pre > 0 else None
        self.args_decode_only = varlen_args(n_pre, n, self.resolved) if n_pre < n else None
        self.kv_bytes = int(w.context_lens.astype("int64").sum()) * hkv * 2 * row_bytes(w)
        self.decode_kv_bytes = int(w.context_lens[n_pre:].astype("int64").sum()) * hkv * 2 * row_bytes(w)
        pos = [(int(L) - int(qn) + i + 1) for L, qn in zip(w.context_lens[:n_pre], w.q_lens[:n_pre]) for i in range(qn)]
        self.prefill_flops = 4 * w.num_q_heads * d * int(sum(max(0, x) for x in pos))


def bench_varlen(args, pa, torch, np, to_dev, lib, stream, sh, check):
    """The packed continuous-batching step (prefill chunks + decode tokens)."""
    from workloads import CONFIG_NAMES, make_config

    w0 = make_config(args.config)
    partition = args.partition if args.partition is not None else -1
    reps = args.replicas or 4
    batches = [VarlenBatch(w0 if r == 0 else make_config(args.config, replica=r), partition, pa, torch, to_dev)
               for r in range(reps)]
    torch.cuda.synchronize()

    def step(b):
        check(lib.paged_kv_slot_mapping(*b.args_slot, sh), "slot mapping")
        check(lib.kv_cache_write(*b.args_write, sh), "cache write")
        check(lib.paged_attention_varlen(*b.args_varlen, sh), "varlen")

    def timed(call, with_events):
        for i in range(args.warmup):
            call(batches[i % reps])
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)] if with_events else None
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        lead_in(torch, stream)
        start.record(stream)
        for i in range(args.steps):
            if with_events:
                evs[i][0].record(stream)
            call(batches[i % reps])
            if with_events:
                evs[i][1].record(stream)
        stop.record(stream)
        torch.cuda.synchronize()
        kern = [a.elapsed_time(b) for a, b in evs] if with_events else None
        timed.last = kern
        return start.elapsed_time(stop) / args.steps, (float(np.mean(kern)) if with_events else None)

    dec = lambda b: check(lib.paged_attention_varlen(*b.args_decode_only, sh), "varlen decode rows")
    pre = lambda b: check(lib.paged_attention_varlen(*b.args_prefill_only, sh), "varlen prefill rows")
    if batches[0].args_decode_only is None:  # every sequence verifies several tokens
        bench_multi_token(args, batches, timed, pre, step, np)
        return
    _, dec_ms = timed(dec, True)
    dec_list = timed.last
    _, pre_ms = timed(pre, True)
    ms_step, _ = timed(step, False)
    step_bytes = float(np.mean([batches[i % reps].kv_bytes for i in range(args.steps)]))
    dec_bytes = float(np.mean([batches[i % reps].decode_kv_bytes for i in range(args.steps)]))
    pre_flops = float(np.mean([batches[i % reps].prefill_flops for i in range(args.steps)]))
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
    pre_tflops = pre_flops / (pre_ms * 1e-3) / 1e12
    cpu = args.cpu_result
    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w0.kv_dtype == "bf16" else f"bf16-q/{w0.kv_dtype}-kv",
        "data": "synthetic",
        "config": {
            "workload": CONFIG_NAMES[args.config],
            "num_seqs": w0.num_seqs,
            "prefill_chunks": int((w0.q_lens > 1).sum()),
            "total_q": w0.total_q,
            "num_q_heads": w0.num_q_heads,
            "num_kv_heads": w0.num_kv_heads,
            "head_dim": w0.head_dim,
            "block_size": w0.block_size,
            "context_lens": resident_lens(batches),
            "partition_tokens": batches[0].resolved,
            "resident_batches": reps,
            "step": "slot mapping + cache write of every new token + paged_attention_varlen (one launch of "
                    "the two-role packed-step kernel: decode rows streamed, prefill tiles on MFMA)",
        },
        "seq_steps_per_s": round(w0.num_seqs / (ms_step * 1e-3), 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "kv_bytes_per_step": int(step_bytes),
        "kv_bytes_note": "mean over the timed steps, which rotate over the resident batches (independently "
                         "seeded, of the same shape); each batch's own bytes are listed",
        "kv_bytes_per_resident_batch": [int(b.kv_bytes) for b in batches],
        "roofline": {
            "kernel": "decode_partition_kernel (1-token rows of the packed batch)",
            "bound": "hbm",
            "achieved": round(dec_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(args.traffic, CONFIG_NAMES[args.config], [i % reps for i in range(args.steps)]),
            "avg_launch_us": round(dec_ms * 1e3, 3),
            "launch_distribution": launch_stats(dec_list),
            "algorithmic_bytes_per_launch": int(dec_bytes),
        },
        "prefill_mfma": {
            "kernel": "prefill rows alone, launched as in the full step: one packed-step launch whose decode "
                      "work-groups find no 1-token row and return",
            "bound": "mfma",
            "achieved": round(pre_tflops, 2),
            "peak": 2500.0,
            "unit": "TFLOP/s",
            "frac": round(pre_tflops / 2500.0, 4),
            "avg_call_us": round(pre_ms * 1e3, 3),
            "flops_per_call": int(pre_flops),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def bench_multi_token(args, batches, timed, call, step, np):
    """A batch whose every sequence attends several new tokens (speculative verification): one
    kernel streams each (sequence, KV head) context once for all its query rows, so the roofline is
    HBM on the same algorithmic KV bytes as a decode step."""
    from workloads import CONFIG_NAMES

    w0 = batches[0].w
    reps = len(batches)
    _, call_ms = timed(call, True)
    call_list = timed.last
    ms_step, _ = timed(step, False)
    step_bytes = float(np.mean([batches[i % reps].kv_bytes for i in range(args.steps)]))
    flops = float(np.mean([batches[i % reps].prefill_flops for i in range(args.steps)]))
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    call_gbs = step_bytes / (call_ms * 1e-3) / 1e9
    cpu = args.cpu_result
    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": CONFIG_NAMES[args.config],
            "num_seqs": w0.num_seqs,
            "tokens_per_seq": int(w0.max_q_len),
            "num_q_heads": w0.num_q_heads,
            "num_kv_heads": w0.num_kv_heads,
            "head_dim": w0.head_dim,
            "block_size": w0.block_size,
            "context_lens": resident_lens(batches),
            "resident_batches": reps,
            "step": "slot mapping + cache write of every new token + paged_attention_varlen (causal among "
                    "the new tokens)",
        },
        "seq_steps_per_s": round(w0.num_seqs / (ms_step * 1e-3), 1),
        "tokens_per_s": round(w0.total_q / (ms_step * 1e-3), 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "kv_bytes_per_step": int(step_bytes),
        "kv_bytes_note": "mean over the timed steps, which rotate over the resident batches (independently "
                         "seeded, of the same shape); each batch's own bytes are listed",
        "kv_bytes_per_resident_batch": [int(b.kv_bytes) for b in batches],
        "roofline": {
            "kernel": "varlen_multiquery_kernel (every row; no decode launch)",
            "bound": "hbm",
            "achieved": round(call_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(call_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(args.traffic, CONFIG_NAMES[args.config], [i % reps for i in range(args.steps)]),
            "avg_launch_us": round(call_ms * 1e3, 3),
            "launch_distribution": launch_stats(call_list),
            "algorithmic_bytes_per_launch": int(step_bytes),
            "mfma_tflops": round(flops / (call_ms * 1e-3) / 1e12, 2),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path needs no second GPU)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import paged_kv_cache_251_amd as pa
    from workloads import CONFIG_NAMES, make_config

    # the oracle's host baseline first: its all-core leg forks workers, before anything touches the GPU
    args.cpu_result = None
    if not args.no_cpu_baseline:
        wc = make_config(args.config)
        args.cpu_result = cpu_baseline(wc, args.cpu_seconds, packed=not wc.is_decode)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lib = pa.lib()

    def to_dev(raw, dtype):
        if dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(raw, np.float32)).to("cuda:0")
        return torch.from_numpy(np.ascontiguousarray(raw, np.uint16).view(np.int16)).to("cuda:0").view(torch.bfloat16)

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def check(st, fn):
        if st != 0:
            raise RuntimeError(f"{fn}: {lib.pa_last_error().decode()}")

    w0 = make_config(args.config)
    if not w0.is_decode:
        bench_varlen(args, pa, torch, np, to_dev, lib, stream, sh, check)
        return
    partition = args.partition if args.partition is not None else (w0.partition_size or -1)
    pool_bytes = w0.num_blocks * w0.num_kv_heads * 16 * 2 * row_bytes(w0)
    reps = args.replicas or max(2, min(8, -(-1_200_000_000 // pool_bytes)))
    t_setup = time.perf_counter()
    batches = [Batch(w0 if r == 0 else make_config(args.config, replica=r), partition, pa, torch, to_dev)
               for r in range(reps)]
    torch.cuda.synchronize()
    print(f"# setup: {reps} resident batches of {CONFIG_NAMES[args.config]} in {time.perf_counter() - t_setup:.1f} s",
          file=sys.stderr, flush=True)

    def step(b, ev=None):
        """Fused step: append + attend in one launch (+ the reduce kernel for split contexts)."""
        if ev is not None:
            ev[0].record(stream)
        check(lib.paged_attention_decode_append(*b.args_append, sh), "decode append")
        if ev is not None:
            ev[1].record(stream)
        if b.split:
            check(lib.paged_attention_decode_reduce(*b.args_reduce, sh), "decode reduce")

    def step_unfused(b, ev=None):
        check(lib.paged_kv_slot_mapping(*b.args_slot, sh), "slot mapping")
        check(lib.kv_cache_write(*b.args_write, sh), "cache write")
        if ev is not None:
            ev[0].record(stream)
        check(lib.paged_attention_decode_partitions(*b.args_parts, sh), "decode partitions")
        if ev is not None:
            ev[1].record(stream)
        if b.split:
            check(lib.paged_attention_decode_reduce(*b.args_reduce, sh), "decode reduce")

    def timed(fn, with_events):
        for i in range(args.warmup):
            fn(batches[i % reps])
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)] if with_events else None
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        lead_in(torch, stream)
        start.record(stream)
        for i in range(args.steps):
            if with_events:
                fn(batches[i % reps], evs[i])
            else:
                fn(batches[i % reps])
        stop.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        kern = [a.elapsed_time(b) for a, b in evs] if with_events else None
        return start.elapsed_time(stop) / args.steps, wall, kern

    # unfused path first (it also warms the clocks), then the roofline loop (a HIP event
    # pair around the partition kernel of every step), then the reported steps, back to
    # back with no events between launches
    fused = batches[0].fused
    main_step = step if fused else step_unfused
    ms_unfused, _, _ = timed(step_unfused, False)
    _, _, kern_ms = timed(main_step, True)
    ms_step, wall, _ = timed(main_step, False)
    # A fused step without a reduce is one launch of the kernel: its average launch duration is the
    # event-timed region over the launches, with no event pair between them (the pairs of the
    # roofline loop add their own few microseconds; their distribution is reported beside it).
    single_launch = fused and not batches[0].split
    kern_avg = ms_step if single_launch else float(np.mean(kern_ms))
    step_bytes = float(np.mean([batches[i % reps].kv_bytes for i in range(args.steps)]))
    seqs = w0.num_seqs
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    kern_gbs = step_bytes / (kern_avg * 1e-3) / 1e9

    traffic = measured_traffic(args.traffic, CONFIG_NAMES[args.config], [i % reps for i in range(args.steps)])

    cpu = args.cpu_result

    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w0.kv_dtype if w0.kv_dtype == w0.q_dtype else f"{w0.q_dtype}-q/{w0.kv_dtype}-kv",
        "data": "synthetic",
        "config": {
            "workload": CONFIG_NAMES[args.config],
            "num_seqs": seqs,
            "num_q_heads": w0.num_q_heads,
            "num_kv_heads": w0.num_kv_heads,
            "head_dim": w0.head_dim,
            "block_size": w0.block_size,
            "context_lens": resident_lens(batches),
            "partition_tokens": batches[0].resolved,
            "resident_batches": reps,
            "step": (("one launch: slot mapping + " + ("quantising " if w0.kv_dtype in SCALED else "") +
                      "cache write of the newest token + decode attention") if fused else
                     f"slot mapping + {w0.kv_dtype.upper()} cache write (quantise) of the newest token + decode "
                     "attention") +
                    (" (split-KV partitions) + the separate reduce kernel" if batches[0].split else ""),
        },
        "seq_steps_per_s": round(seqs / (ms_step * 1e-3), 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "kv_bytes_per_step": int(step_bytes),
        "kv_bytes_note": "mean over the timed steps, which rotate over the resident batches (independently "
                         "seeded, of the same shape); each batch's own bytes are listed",
        "kv_bytes_per_resident_batch": [int(b.kv_bytes) for b in batches],
        "unfused": None if not fused else {
            "ms_per_step": round(ms_unfused, 5),
            "GB_per_s": round(step_bytes / (ms_unfused * 1e-3) / 1e9, 2),
            "calls": "paged_kv_slot_mapping + kv_cache_write + decode partitions" +
                     (" + separate reduce kernel" if batches[0].split else "")},
        "wall_s": round(wall, 4),
        "roofline": {
            "kernel": decode_kernel_name(w0) + (" (append mode" if fused else " (") + f", {w0.kv_dtype.upper()} pool)",
            "bound": "hbm",
            "achieved": round(kern_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(kern_avg * 1e3, 3),
            "avg_launch_from": ("event pair around the timed region of back-to-back steps, each one launch of the "
                                "kernel" if single_launch else "event pair around every launch of the kernel"),
            "launch_distribution": launch_stats(kern_ms),
            "algorithmic_bytes_per_launch": int(step_bytes),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def decode_kernel_name(w) -> str:
    """The partition kernel a decode call launches: groups of 8 or 16 query heads per KV head over
    a bf16 or E5M2 cache run on MFMA, every other shape on the vector kernel."""
    return "decode_mfma_kernel" if w.gqa_group in (8, 16) and w.kv_dtype in ("bf16", "e5m2") else "decode_partition_kernel"


# Sources each measured kernel is built and launched from: its traffic figure only counts while
# they are unchanged.
KERNEL_SOURCES = {
    "decode": ("decode.hip", "decode_body.hpp", "multiquery.hip", "pa_device.hpp", "pa_launch.hpp", "api.cpp"),
    "multiquery": ("multiquery.hip", "pa_device.hpp", "pa_launch.hpp", "api.cpp"),
}


def kernel_family(workload: str) -> str:
    return "multiquery" if workload.startswith("llama3_8b_spec_verify") else "decode"


def kernel_source_digest(family: str) -> str:
    """sha256 over the sources of one kernel family: measured traffic only counts for the
    sources it was measured on."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_251_amd", "csrc")
    for name in KERNEL_SOURCES[family]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(path, workload, replicas=None):
    """HBM bytes per launch of the dominant kernel for this workload, from the committed
    rocprofv3 counter summary, or None when it is missing or was taken on other sources.  The
    summary holds the bytes of each resident batch (they differ in size); `replicas` lists the
    batch of every timed step, and the result is their mean, like the algorithmic bytes."""
    if not path or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    entry = rec.get("workloads", {}).get(workload)
    if entry is None or entry.get("source_sha256") != kernel_source_digest(kernel_family(workload)):
        return None
    by_rep = entry.get("hbm_bytes_by_replica")
    if replicas and by_rep and all(0 <= r < len(by_rep) and by_rep[r] for r in replicas):
        return int(round(sum(by_rep[r] for r in replicas) / len(replicas)))
    return entry.get("hbm_bytes_per_launch")


def _compact(w, sel):
    """Block tables of the selected sequences renumbered onto a pool that holds only their blocks
    (so a pass's oracle pools stay small): (tables, num_blocks)."""
    import numpy as np

    bt = np.asarray(w.block_tables)
    used = np.unique(bt[sel][bt[sel] >= 0])
    remap = np.full(max(w.num_blocks, 1), -1, np.int64)
    remap[used] = np.arange(used.size)
    tables = np.where(bt >= 0, remap[np.clip(bt, 0, None)], -1).astype(np.int32)
    tables[[s for s in range(w.num_seqs) if s not in set(sel)]] = -1
    return tables, max(int(used.size), 1)


def _oracle_passes(w, seqs, budget_s, packed):
    """Time the oracle (as it stands) on the host: each pass takes the next 8 of ``seqs`` through
    the oracle's slot mapping, cache write of the step's new tokens and paged attention (decode, or
    the causal packed step), until the budget is spent.  The pass's history (the tokens cached
    before the step) is written untimed.  Returns (sequence-steps, KV bytes, seconds timed)."""
    import numpy as np

    import oracle
    from workloads import POISON_BITS, queries, write_plan

    q = queries(w)
    scaled = w.kv_dtype in SCALED
    done_seqs, done_bytes, t_used, i0 = 0, 0, 0.0, 0
    while t_used < budget_s:
        sel = [seqs[(i0 + i) % len(seqs)] for i in range(min(8, len(seqs)))]
        i0 += len(sel)
        tables, nb = _compact(w, sel)
        if scaled:  # the oracle's scaled pool: dequantised rows (code value * scale), float64
            pk = np.full((nb, w.block_size, w.num_kv_heads, w.head_dim), np.nan)
        else:
            pk = oracle.new_pool(nb, w.block_size, w.num_kv_heads, w.head_dim, w.kv_dtype, POISON_BITS[w.kv_dtype])
        pv = pk.copy()

        def write(pool, rows, slots):
            if scaled:
                quant, dequant = ((oracle.quantize_int8, oracle.dequantize_int8) if w.kv_dtype == "int8" else
                                  (oracle.quantize_e4m3, oracle.dequantize_e4m3))
                codes, scales = quant(oracle.decode_storage(rows, w.src_dtype).astype(np.float32))
                keep = slots >= 0
                pool[slots[keep] // w.block_size, slots[keep] % w.block_size] = dequant(codes[keep], scales[keep])
            else:
                oracle.cache_write(pool, rows, slots, w.src_dtype, w.kv_dtype, w.block_size)

        hist = write_plan(w, "cached", sel)
        hs = oracle.slot_mapping(tables, hist.counts, hist.end_pos, w.block_size)
        write(pk, hist.k, hs)
        write(pv, hist.v, hs)
        new = write_plan(w, "new", sel)
        t0 = time.perf_counter()
        ns = oracle.slot_mapping(tables, new.counts, new.end_pos, w.block_size)
        write(pk, new.k, ns)
        write(pv, new.v, ns)
        if packed:
            oracle.paged_varlen(pk, pv, w.kv_dtype, q, "bf16", w.cu_seqlens_q, tables, w.context_lens, w.block_size,
                                w.scale, causal=True, seqs=sel)
        else:
            oracle.paged_decode(pk, pv, "f64" if scaled else w.kv_dtype, q, w.q_dtype, tables, w.context_lens,
                                w.block_size, w.scale, seqs=sel)
        t_used += time.perf_counter() - t0
        done_seqs += len(sel)
        done_bytes += int(w.context_lens[sel].astype(np.int64).sum()) * w.num_kv_heads * 2 * row_bytes(w)
    return done_seqs, done_bytes, t_used


def _oracle_worker(arg):
    from threadpoolctl import threadpool_limits

    w, seqs, budget_s, packed = arg
    with threadpool_limits(limits=1):
        return _oracle_passes(w, seqs, budget_s, packed)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


MAX_CPU_WORKERS = 16  # the host share of one GPU on the measuring boxes


def cpu_baseline(w, budget_s, packed=False):
    """The oracle on the host's cores, twice: one process with one BLAS thread, then one forked
    worker process per affinity core (at most 16), each timing the oracle on its own share of the
    batch's sequences.  The all-core rate is the sum of the workers' rates over their timed passes.
    Runs before the GPU is initialised (the workers are forked)."""
    import multiprocessing

    cores = max(1, min(len(os.sched_getaffinity(0)), MAX_CPU_WORKERS))
    half = budget_s / 2
    n1, b1, t1 = _oracle_worker((w, list(range(w.num_seqs)), half, packed))
    shards = [list(range(i, w.num_seqs, cores)) for i in range(min(cores, w.num_seqs))]
    with multiprocessing.get_context("fork").Pool(len(shards)) as pool:
        res = pool.map(_oracle_worker, [(w, sh, half, packed) for sh in shards])
    rate_b = sum(b / t for _, b, t in res)
    rate_s = sum(n / t for n, _, t in res)
    what = ("slot mapping, cache write of the new tokens, causal float64 attention" if packed else
            "slot mapping, cache write of the newest token, float64 attention")
    return {
        "value": round(rate_b / 1e9, 4),
        "unit": "GB/s",
        "seq_steps_per_s": round(rate_s, 3),
        "cores": len(shards),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"{sum(n for n, _, _ in res)} sequence-steps of the {w.num_seqs}-sequence timed workload "
                  f"({what} each), split over {len(shards)} worker processes with one BLAS thread each, "
                  f"{half:.0f} s of timed passes per worker; rate = sum of the workers' rates",
        "single_core": {"value": round(b1 / t1 / 1e9, 4), "unit": "GB/s", "seq_steps_per_s": round(n1 / t1, 3),
                        "cores": 1, "sample": f"{n1} sequence-steps in {t1:.1f} s, one process, one BLAS thread"},
    }


if __name__ == "__main__":
    main()
