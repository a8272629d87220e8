"""Block allocator of a paged KV cache, written out plainly.  TEST
INFRASTRUCTURE ONLY (see the package docstring).

The pages keep the cache in fixed-size blocks handed out on demand as tokens
are generated, with waste bounded by the last, partly filled block ("TensorRT-LLM
Guide: High-Throughput GPU Inference Engine", section "2. Paged KV Cache &
Memory Virtualization"), and reuse blocks across requests that share a prefix
("Lesson 13.17 TensorRT-LLM: NVIDIA's Optimized Inference Engine", section
"The paged KV cache, in-flight batching and CUDA graphs").  Reading taken
where the pages are silent: a block shared by several sequences is copied to
a fresh block before one of them appends to it (copy on write), so no
sequence sees another's appended token; when every holder appends in the same
step, the last holder in batch order keeps the block.  The order in which
free blocks and sequence ids are handed out is the library's stated one (a
stack of free blocks that starts 0, 1, 2, ...; the lowest free sequence id),
so block ids can be compared exactly.
"""
from __future__ import annotations


class AllocError(Exception):
    def __init__(self, kind: str, msg: str):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind            # "invalid" or "oom"


class BlockAllocator:
    def __init__(self, num_blocks: int, block_size: int, max_seqs: int):
        if num_blocks < 1 or block_size < 1 or max_seqs < 1:
            raise AllocError("invalid", "sizes must be >= 1")
        self.block_size = block_size
        self.free = list(range(num_blocks - 1, -1, -1))      # stack: pop() -> 0 first
        self.ref = [0] * num_blocks
        self.max_seqs = max_seqs
        self.seqs = {}                                        # id -> [length, [blocks]]

    def _pop(self) -> int:
        b = self.free.pop()
        self.ref[b] = 1
        return b

    def _new_id(self) -> int:
        for i in range(self.max_seqs):
            if i not in self.seqs:
                return i
        raise AllocError("oom", "no sequence id")

    def _live(self, s: int):
        if s not in self.seqs:
            raise AllocError("invalid", f"sequence {s} is not live")
        return self.seqs[s]

    def add(self, length: int) -> int:
        if length < 0:
            raise AllocError("invalid", "length < 0")
        sid = self._new_id()
        nb = -(-length // self.block_size)
        if nb > len(self.free):
            raise AllocError("oom", "blocks")
        self.seqs[sid] = [length, [self._pop() for _ in range(nb)]]
        return sid

    def fork(self, parent: int) -> int:
        length, blocks = self._live(parent)
        sid = self._new_id()
        for b in blocks:
            self.ref[b] += 1
        self.seqs[sid] = [length, list(blocks)]
        return sid

    def release(self, s: int) -> None:
        _, blocks = self._live(s)
        for b in reversed(blocks):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.seqs[s]

    def prepare_step(self, seq_ids, max_blocks: int, max_copies: int):
        """Tables, lengths, positions and copy pairs of one step, or an error
        with nothing changed."""
        ids = [int(s) for s in seq_ids]
        if len(set(ids)) != len(ids):
            raise AllocError("invalid", "repeated id")
        fresh = 0
        writers = {}
        for s in ids:
            length, blocks = self._live(s)
            if -(-(length + 1) // self.block_size) > max_blocks:
                raise AllocError("invalid", "outgrows the table")
            if length % self.block_size == 0:
                fresh += 1
            else:
                b = blocks[length // self.block_size]
                if self.ref[b] > 1:
                    writers[b] = writers.get(b, 0) + 1
        cow = sum(k - (1 if self.ref[b] == k else 0) for b, k in writers.items())
        if cow > max_copies:
            raise AllocError("invalid", "copies")
        if fresh + cow > len(self.free):
            raise AllocError("oom", "blocks")
        tables, lens, pos, copies = [], [], [], []
        for s in ids:
            rec = self.seqs[s]
            length, blocks = rec
            if length % self.block_size == 0:
                blocks.append(self._pop())
            else:
                j = length // self.block_size
                b = blocks[j]
                if self.ref[b] > 1:
                    dst = self._pop()
                    copies.append((b, dst))
                    self.ref[b] -= 1
                    blocks[j] = dst
            rec[0] = length + 1
            tables.append(blocks + [-1] * (max_blocks - len(blocks)))
            lens.append(length + 1)
            pos.append(length)
        return tables, lens, pos, copies
