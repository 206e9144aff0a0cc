"""Reference step scheduler -- TEST INFRASTRUCTURE, not part of the product path.

Plain Python over the reference block manager, written for reading.  It follows the pages:
  * Colossal-Inference release post, "连续批量化算法 (Continuous Batching)": prefill and decode
    are computed as separate steps over unpadded input; a prefill step is run once the inputs
    that need prefill reach a set ratio, so that most steps are decode steps.
  * LLM inference optimisation overview, 2.4 "服务": step-level scheduling over a Running and a
    Waiting queue -- a finished sequence leaves Running and waiting ones take its place -- and
    dynamic batching: after each step the Running queue grows or shrinks with the memory left.
  * The same overview, 2.1.2 "Paged Attention": block-granular accounting tells how many more
    blocks fit, which is what keeps the pool from overflowing; max_num_batch_tokens bounds the
    tokens of one batch.
and the readings the library's header states where the pages are silent: the ratio compares
|Waiting| with |Running|; admission is in FIFO order and stops at the first request that does
not fit (Running full, the step's known tokens over max_batch_tokens -- the first admitted
always fits -- or the pool unable to hold it); an empty prefill step becomes a decode step; a
decode step that cannot get a block preempts the most recently admitted running sequence,
whose request goes back to the head of Waiting with every token it knows.
"""
from __future__ import annotations

from collections import deque

from .block_manager import OutOfBlocks, RefBlockManager

IDLE, PREFILL, DECODE = 0, 1, 2


class RefScheduler:
    def __init__(self, manager: RefBlockManager, max_running: int, max_batch_tokens: int, prefill_ratio: float,
                 max_blocks_per_seq: int):
        self.bm = manager
        self.max_running = max_running
        self.max_batch_tokens = max_batch_tokens
        self.ratio = prefill_ratio
        self.max_blocks = max_blocks_per_seq
        self.req = {}          # id -> dict(tokens, max_new, generated)
        self.waiting = deque()
        self.running = []      # admission order
        self.pending = []      # the last step's sequences, until commit
        self.finished = 0
        self.preemptions = 0

    def add_request(self, rid, prompt, max_new_tokens):
        assert rid not in self.req and len(prompt) >= 1 and max_new_tokens >= 1
        most = len(prompt) + max_new_tokens - 1
        if most > self.max_batch_tokens or -(-most // self.bm.B) > min(self.max_blocks, self.bm.num_blocks):
            raise ValueError("request too long")
        self.req[rid] = dict(tokens=list(prompt), max_new=max_new_tokens, generated=0)
        self.waiting.append(rid)

    def _table(self, rid):
        blocks, _ = self.bm.block_table(rid)
        return blocks + [-1] * (self.max_blocks - len(blocks))

    def step(self):
        """Returns dict(kind, seq_ids, q_lens, context_lens, tables, input_tokens, copies, preempted)."""
        assert not self.pending
        out = dict(kind=IDLE, seq_ids=[], q_lens=[], context_lens=[], tables=[], input_tokens=[], copies=[],
                   preempted=[])
        room = len(self.running) < self.max_running
        ratio_ok = not self.running or len(self.waiting) >= self.ratio * len(self.running)
        if self.waiting and room and ratio_ok:
            known = 0
            while self.waiting and len(self.running) < self.max_running:
                rid = self.waiting[0]
                toks = self.req[rid]["tokens"]
                if out["seq_ids"] and known + len(toks) > self.max_batch_tokens:
                    break
                try:
                    cached = self.bm.add_sequence(rid, len(toks), toks)
                except OutOfBlocks:
                    break
                self.waiting.popleft()
                self.running.append(rid)
                known += len(toks)
                out["seq_ids"].append(rid)
                out["q_lens"].append(len(toks) - cached)
                out["context_lens"].append(len(toks))
                out["input_tokens"] += toks[cached:]
                out["tables"].append(self._table(rid))
            if out["seq_ids"]:
                out["kind"] = PREFILL
                self.pending = list(out["seq_ids"])
                return out
        i = 0
        while i < len(self.running):
            rid = self.running[i]
            try:
                out["copies"] += self.bm.append(rid, 1, [self.req[rid]["tokens"][-1]])
                i += 1
            except OutOfBlocks:
                victim = self.running.pop()
                self.bm.free_sequence(victim)
                self.waiting.appendleft(victim)
                out["preempted"].append(victim)
                self.preemptions += 1
        for rid in self.running:
            toks = self.req[rid]["tokens"]
            out["seq_ids"].append(rid)
            out["q_lens"].append(1)
            out["context_lens"].append(len(toks))
            out["input_tokens"].append(toks[-1])
            out["tables"].append(self._table(rid))
        out["kind"] = DECODE if self.running else IDLE
        self.pending = list(out["seq_ids"])
        return out

    def commit(self, next_tokens, finished=None):
        assert len(next_tokens) == len(self.pending)
        done = set()
        for i, rid in enumerate(self.pending):
            r = self.req[rid]
            r["tokens"].append(int(next_tokens[i]))
            r["generated"] += 1
            if (finished is not None and finished[i]) or r["generated"] >= r["max_new"]:
                self.bm.free_sequence(rid)
                del self.req[rid]
                done.add(rid)
                self.finished += 1
        self.running = [rid for rid in self.running if rid not in done]
        self.pending = []

    def stats(self):
        return len(self.waiting), len(self.running), self.finished, self.preemptions
