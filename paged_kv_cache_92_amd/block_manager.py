"""Host-side KV block manager: free list, reference counts, copy-on-write.

This is the bookkeeping that produces the integer inputs of the GPU path —
block tables, slot mappings and copy-on-write (src, dst) pairs.  It holds no
attention arithmetic and no device memory.

Behaviour follows the pages:

* Fixed-size blocks of ``block_size`` token slots, taken from a pool of free
  physical blocks; a sequence's block table maps logical block i to a
  physical block ("vLLM — KV Cache와 PagedAttention 완전 해부", hrletsgo.me,
  step 5).
* Blocks fill left to right and a new physical block is taken only when the
  last one is full ("Sparse Computation and Memory Management for Efficient
  LLM Inference", pyy0715.github.io, section "Memory Allocation
  Pseudocode"), so a sequence of n tokens holds ceil(n / B) blocks.
* When the pool cannot cover a request, allocation fails and nothing is
  taken: the caller (a scheduler) would preempt ("[vLLM] PagedAttention",
  blog.secrett2633.cloud, section "블록 할당: allocate_slots" returns None).
  Here that is ``OutOfBlocks``.
* Shared blocks carry a reference count; writing into a block whose count
  exceeds one first copies it to a new block, decrements the old count and
  repoints the writer's table (same pyy0715.github.io page, section
  "Copy-on-Write"; hrletsgo.me step 9).
* A finished sequence returns its blocks (hrletsgo.me step 7.7).
* Under a sliding window of W tokens, blocks that hold only positions before
  the window of the sequence's newest token are released before new ones are
  taken, as an OS pages out frames (blog.secrett2633.cloud, section "블록
  할당: allocate_slots", remove_skipped_blocks); their table entries become
  ``NULL_BLOCK``.

A slot number is ``physical_block * block_size + offset``.
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

import numpy as np


NULL_BLOCK = -1   # table entry of a block released from before a sliding window


class OutOfBlocks(RuntimeError):
    """Raised when the free list cannot cover an allocation (the pages' ``None``)."""


@dataclass
class SeqState:
    seq_id: int
    block_table: list[int] = field(default_factory=list)
    num_tokens: int = 0


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        """``free_order`` is the order in which physical blocks leave the free list
        (a seeded permutation scatters a sequence's blocks across the pool)."""
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = range(num_blocks) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the pool")
        self._free = deque(order)
        self.ref_count = np.zeros(num_blocks, dtype=np.int64)
        self._seqs: dict[int, SeqState] = {}
        self._next_id = 0

    # -- pool ---------------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self._free)

    def _take(self) -> int:
        if not self._free:
            raise OutOfBlocks("no free KV block")
        b = self._free.popleft()
        self.ref_count[b] = 1
        return b

    def _release(self, b: int):
        if b == NULL_BLOCK:
            return
        self.ref_count[b] -= 1
        if self.ref_count[b] < 0:
            raise AssertionError(f"block {b} released more times than it was held")
        if self.ref_count[b] == 0:
            self._free.append(b)

    # -- sequences ------------------------------------------------------------
    def new_sequence(self) -> int:
        sid = self._next_id
        self._next_id += 1
        self._seqs[sid] = SeqState(sid)
        return sid

    def seq(self, sid: int) -> SeqState:
        return self._seqs[sid]

    def fork(self, parent: int) -> int:
        """A new sequence sharing every block of ``parent`` (reference counts + 1)."""
        p = self._seqs[parent]
        sid = self.new_sequence()
        child = self._seqs[sid]
        child.block_table = list(p.block_table)
        child.num_tokens = p.num_tokens
        for b in p.block_table:
            if b != NULL_BLOCK:
                self.ref_count[b] += 1
        return sid

    def blocks_needed(self, sid: int, n: int) -> int:
        """Fresh blocks that appending n tokens takes, copy-on-write copies included."""
        s = self._seqs[sid]
        B = self.block_size
        have = len(s.block_table)
        need = -(-(s.num_tokens + n) // B) - have
        cow = 0
        if n > 0 and s.num_tokens % B != 0 and self.ref_count[s.block_table[-1]] > 1:
            cow = 1
        return need + cow

    def append_tokens(self, sid: int, n: int):
        """Allocate slots for n new tokens of sequence ``sid``.

        Returns ``(slots, copies)``: int64 slot numbers of the n tokens in order,
        and a list of (src, dst) block copies that must run before those tokens
        are written.  Either the whole request succeeds or ``OutOfBlocks`` is
        raised with the manager unchanged.
        """
        s = self._seqs[sid]
        B = self.block_size
        if n < 0:
            raise ValueError("n must be >= 0")
        if self.blocks_needed(sid, n) > self.num_free:
            raise OutOfBlocks(f"sequence {sid} needs {self.blocks_needed(sid, n)} blocks, "
                              f"{self.num_free} free")
        copies = []
        slots = np.empty(n, dtype=np.int64)
        i = 0
        off = s.num_tokens % B
        if n > 0 and off != 0:
            # Tokens that fill the partially used last block.  Only the first of
            # them can meet a shared block: copy-on-write makes it private.
            logical = s.num_tokens // B
            phys = s.block_table[logical]
            if self.ref_count[phys] > 1:
                new_phys = self._take()
                copies.append((phys, new_phys))
                self.ref_count[phys] -= 1
                s.block_table[logical] = new_phys
            k = min(n, B - off)
            slots[:k] = s.block_table[logical] * B + off + np.arange(k)
            s.num_tokens += k
            i = k
        while i < n:
            # The last block is full (or there is none): take a new one.
            b = self._take()
            s.block_table.append(b)
            k = min(B, n - i)
            slots[i:i + k] = b * B + np.arange(k)
            s.num_tokens += k
            i += k
        return slots, copies

    def remove_skipped_blocks(self, sid: int, window: int) -> int:
        """Release the blocks of ``sid`` that hold only positions before
        ``num_tokens - window`` (outside the window of the newest token and of
        every later one); returns how many were released."""
        s = self._seqs[sid]
        if window <= 0:
            return 0
        first = max(0, s.num_tokens - window) // self.block_size
        n = 0
        for i in range(min(first, len(s.block_table))):
            if s.block_table[i] != NULL_BLOCK:
                self._release(s.block_table[i])
                s.block_table[i] = NULL_BLOCK
                n += 1
        return n

    def free_sequence(self, sid: int):
        s = self._seqs.pop(sid)
        for b in s.block_table:
            self._release(b)

    def block_table_array(self, sids, max_blocks: int, pad: int) -> np.ndarray:
        """int32 [len(sids)][max_blocks]; entries past a sequence's blocks hold ``pad``."""
        out = np.full((len(sids), max_blocks), pad, dtype=np.int32)
        for r, sid in enumerate(sids):
            bt = self._seqs[sid].block_table
            if len(bt) > max_blocks:
                raise ValueError(f"sequence {sid} holds {len(bt)} blocks > {max_blocks}")
            out[r, :len(bt)] = bt
        return out

    def wasted_slots(self) -> int:
        """Allocated-but-empty token slots over live sequences (each block counted once)."""
        held = {b for s in self._seqs.values() for b in s.block_table if b != NULL_BLOCK}
        used = np.zeros(self.num_blocks, dtype=np.int64)
        for s in self._seqs.values():
            for i, b in enumerate(s.block_table):
                if b == NULL_BLOCK:
                    continue
                fill = min(self.block_size, s.num_tokens - i * self.block_size)
                used[b] = max(used[b], fill)
        return int(sum(self.block_size - used[b] for b in held))
