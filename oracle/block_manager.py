"""Reference block manager -- TEST INFRASTRUCTURE, not part of the product path.

Plain Python with linear scans, written for reading, not speed.  It follows the pages:
  * Colossal-Inference release post, "分块式KV缓存 (BlockedKeyValueCache)": a sequence's
    cache is cut into fixed-size blocks taken from the pool as its tokens arrive; only its last
    block is partly empty.
  * LLM inference optimisation overview, 2.1.2 "Paged Attention": the pool is reserved up
    front; a table maps logical blocks to physical ones; several logical blocks may name one
    physical block; a block is in use while its reference count is one or more and is freed
    when it drops to zero (the page's "> 1" read as ">= 1").
  * Taco-LLM article, "使用 Prefix Cache 技术降低 TTFT": earlier prompts' cache is kept as a
    prefix tree and the matching part of a new prompt is taken from it instead of recomputed.
and the readings the library's header states where the pages are silent: the lowest free
block is taken first; a full block of a sequence given its token ids is registered in the
tree under (parent block, its tokens) if its parent is registered and the key is new; a new
prompt reuses its longest registered chain, up to (n - 1) // block_size blocks; a block whose
count drops to zero is free unless registered, and registered blocks are evicted when needed,
least recently released leaf first (ties: deeper first, then lower id); appending to a
sequence whose partly filled last block is shared first moves it to a new block (copy on
write); a call that cannot get its blocks changes nothing.
"""
from __future__ import annotations


class OutOfBlocks(Exception):
    pass


class RefBlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        assert num_blocks > 0 and block_size > 0
        self.B = block_size
        self.num_blocks = num_blocks
        self.count = [0] * num_blocks     # reference counts
        self.key = {}                     # registered block -> (parent, tokens)
        self.depth = {}                   # registered block -> its index in the sequence
        self.released = [0] * num_blocks  # time the count last dropped to zero
        self.clock = 0
        self.seqs = {}                    # id -> dict(blocks, n, tracked, chain, tail)

    # -- the pool ---------------------------------------------------------------------------
    def _free(self):
        return [b for b in range(self.num_blocks) if self.count[b] == 0 and b not in self.key]

    def _idle_registered(self):
        return [b for b in self.key if self.count[b] == 0]

    def _children(self, b):
        return [c for c, (parent, _) in self.key.items() if parent == b]

    def _available(self):
        return len(self._free()) + len(self._idle_registered())

    def _take(self):
        free = self._free()
        if free:
            b = min(free)
        else:
            leaves = [c for c in self._idle_registered() if not self._children(c)]
            b = min(leaves, key=lambda c: (self.released[c], -self.depth[c], c))
            del self.key[b]
            del self.depth[b]
        self.count[b] = 1
        return b

    def _lookup(self, parent, tokens):
        for b, k in self.key.items():
            if k == (parent, tuple(tokens)):
                return b
        return None

    def _filled(self, seq, index, tokens):
        if not seq["tracked"] or not seq["chain"]:
            return
        parent = -1 if index == 0 else seq["blocks"][index - 1]
        if self._lookup(parent, tokens) is not None:
            seq["chain"] = False
            return
        b = seq["blocks"][index]
        self.key[b] = (parent, tuple(tokens))
        self.depth[b] = index

    def _extend(self, seq, tokens, n):
        for i in range(n):
            if seq["n"] % self.B == 0:
                seq["blocks"].append(self._take())
            if seq["tracked"]:
                seq["tail"].append(tokens[i])
            seq["n"] += 1
            if seq["n"] % self.B == 0:
                self._filled(seq, len(seq["blocks"]) - 1, seq["tail"])
                seq["tail"] = []

    # -- operations -------------------------------------------------------------------------
    def add_sequence(self, sid, n, tokens=None):
        assert sid not in self.seqs and n >= 0
        matched = []
        if tokens is not None and n > 0:
            parent = -1
            for i in range((n - 1) // self.B):
                b = self._lookup(parent, tokens[i * self.B:(i + 1) * self.B])
                if b is None:
                    break
                matched.append(b)
                parent = b
        needed = -(-n // self.B) - len(matched)
        if needed > self._available() - sum(1 for b in matched if self.count[b] == 0):
            raise OutOfBlocks()
        seq = dict(blocks=[], n=0, tracked=tokens is not None, chain=True, tail=[])
        for b in matched:
            self.count[b] += 1
            seq["blocks"].append(b)
        seq["n"] = len(matched) * self.B
        first = seq["n"]
        self._extend(seq, None if tokens is None else list(tokens[first:]), n - first)
        self.seqs[sid] = seq
        return first

    def append(self, sid, n, tokens=None):
        seq = self.seqs[sid]
        assert n >= 0 and (n == 0 or seq["tracked"] == (tokens is not None))
        if n == 0:
            return []
        partial = seq["n"] % self.B != 0
        cow = partial and self.count[seq["blocks"][-1]] > 1
        needed = -(-(seq["n"] + n) // self.B) - len(seq["blocks"]) + (1 if cow else 0)
        if needed > self._available():
            raise OutOfBlocks()
        copies = []
        if cow:
            old = seq["blocks"][-1]
            new = self._take()
            self.count[old] -= 1
            seq["blocks"][-1] = new
            copies.append((old, new))
        self._extend(seq, None if tokens is None else list(tokens), n)
        return copies

    def fork(self, parent, child):
        assert parent in self.seqs and child not in self.seqs
        src = self.seqs[parent]
        self.seqs[child] = dict(blocks=list(src["blocks"]), n=src["n"], tracked=src["tracked"], chain=src["chain"],
                                tail=list(src["tail"]))
        for b in src["blocks"]:
            self.count[b] += 1

    def free_sequence(self, sid):
        seq = self.seqs.pop(sid)
        self.clock += 1
        for b in seq["blocks"]:
            self.count[b] -= 1
            if self.count[b] == 0:
                self.released[b] = self.clock

    def block_table(self, sid):
        seq = self.seqs[sid]
        return list(seq["blocks"]), seq["n"]

    def stats(self):
        return len(self._free()), len(self.key), sum(1 for c in self.count if c > 0)
