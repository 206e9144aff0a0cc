"""The hot path captured in a HIP graph (needs an MI355X).

Serving loops capture a decode step once and replay it.  Each case below captures the library
calls of one step (no torch work inside the capture; the library records no memset and
allocates nothing), replays the graph several times with eager library work and host
synchronisation in between, and checks every replay bit for bit against the same calls run
eagerly.  Cases: the fused append step (whole contexts, longest-first order), the split-KV
decode with its reduce, the packed prefill + decode step, and the INT8 write + decode.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_251_amd as pa
from gpu_harness import DEV, DeviceBatch, to_device
from workloads import make_config, make_workload, write_plan

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32) if t.dtype == torch.float32 else t


def _replay_and_compare(step, outs, eager_noise):
    """Run step eagerly (reference), capture it, replay 3 times with eager work between."""
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream (first-use host caches)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        for o in outs:
            o.zero_()
        eager_noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, want in zip(outs, ref):
            assert torch.equal(_bits(o), _bits(want)), f"replay {r}"


def _noise():
    """Eager library work on another batch between replays."""
    w = make_workload([40, 7], num_q_heads=4, num_kv_heads=2, head_dim=64, q_dtype="bf16", seed=5)
    b = DeviceBatch(w)
    b.decode(0)


def test_graph_fused_append_step():
    w = make_config(2)
    b = DeviceBatch(w, phases=("cached",))
    plan = write_plan(w, "new")
    k, v = to_device(plan.k, "bf16"), to_device(plan.v, "bf16")
    out = torch.empty_like(b.q)
    ws = pa.alloc_workspace(max(pa.workspace_size(w.num_seqs, w.num_kv_heads, w.gqa_group, w.head_dim,
                                                  w.max_context_len, -1), 256), DEV)

    def step():
        pa.paged_attention_decode_append(b.q, k, v, b.pk, b.pv, b.tables, b.lens, w.max_context_len, w.scale,
                                         partition_size=-1, out=out, workspace=ws)

    _replay_and_compare(step, [out], _noise)


def test_graph_split_decode_with_reduce():
    w = make_workload([3000, 1, 700, 2049], num_q_heads=16, num_kv_heads=2, head_dim=128, q_dtype="bf16", seed=12)
    b = DeviceBatch(w)
    out = torch.empty_like(b.q)
    ws = pa.alloc_workspace(pa.workspace_size(w.num_seqs, w.num_kv_heads, w.gqa_group, w.head_dim,
                                              w.max_context_len, 256), DEV)

    def step():
        pa.paged_attention_decode(b.q, b.pk, b.pv, b.tables, b.lens, w.max_context_len, w.scale, partition_size=256,
                                  out=out, workspace=ws)

    _replay_and_compare(step, [out], _noise)


def test_graph_packed_step():
    w = make_config(5)
    b = DeviceBatch(w, phases=("cached",))
    plan = write_plan(w, "new")
    k, v = to_device(plan.k, "bf16"), to_device(plan.v, "bf16")
    cu = torch.from_numpy(w.cu_seqlens_q).to(DEV)
    cu_new = torch.from_numpy(plan.cu).to(DEV)
    end = torch.from_numpy(plan.end_pos).to(DEV)
    slots = torch.empty(plan.num_tokens, dtype=torch.int32, device=DEV)
    out = torch.empty_like(b.q)
    ws = pa.alloc_workspace(max(pa.workspace_size(w.num_seqs, w.num_kv_heads, w.gqa_group, w.head_dim,
                                                  w.max_context_len, -1), 256), DEV)

    def step():
        pa.slot_mapping(cu_new, end, b.tables, plan.num_tokens, w.num_blocks, 16, out=slots)
        pa.kv_cache_write(k, v, b.pk, b.pv, slots)
        pa.paged_attention_varlen(b.q, b.pk, b.pv, cu, b.lens, b.tables, w.max_q_len, w.max_context_len, w.scale,
                                  causal=True, out=out, workspace=ws)

    _replay_and_compare(step, [out, slots], _noise)


def test_graph_int8_write_and_decode():
    w = make_workload([900, 33, 0, 1600], num_q_heads=8, num_kv_heads=2, head_dim=128, q_dtype="bf16",
                      src_dtype="bf16", kv_dtype="int8", seed=21)
    b = DeviceBatch(w, phases=("cached",))
    plan = write_plan(w, "new")
    k, v = to_device(plan.k, "bf16"), to_device(plan.v, "bf16")
    cu_new = torch.from_numpy(plan.cu).to(DEV)
    end = torch.from_numpy(plan.end_pos).to(DEV)
    slots = torch.empty(plan.num_tokens, dtype=torch.int32, device=DEV)
    out = torch.empty_like(b.q)

    def step():
        pa.slot_mapping(cu_new, end, b.tables, plan.num_tokens, w.num_blocks, 16, out=slots)
        pa.kv_cache_write(k, v, b.pk, b.pv, slots)
        pa.paged_attention_decode(b.q, b.pk, b.pv, b.tables, b.lens, w.max_context_len, w.scale, partition_size=0,
                                  out=out)

    _replay_and_compare(step, [out, slots], _noise)
