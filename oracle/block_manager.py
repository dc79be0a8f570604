"""Reference model of the paged KV block manager (test infrastructure, part of the oracle).

Only ``tests/`` may use it. It restates, step by step, the allocation rules of
"PagedAttention and KV Cache Management" (blog.sejan.dev):

* section "How Block Paging Operates During Generation", item 1 (on-demand allocation: a prompt
  of n tokens gets ceil(n / B) blocks) and item 2 (boundary allocation: a new block is popped from
  the free list only when a token crosses a multiple of B);
* section "Advanced Memory Sharing: Prefix Caching & Copy-on-Write", part 2 (fork shares the
  parent's blocks and raises their reference counts; a write into a shared block first copies it
  into a fresh block, lowers the shared block's count and repoints the writer's table);
* section "Hands-On Implementation: Building a PagedAttention Block Allocator in Python" for the
  order conventions its printed run depends on: the free list is popped from the front, freed
  blocks go to its back, and an empty free list is an out-of-memory error.

Reading where the prose and the listing differ: a copy is made only when the new token is written
into a shared block (the prose). The listing also copies a full shared last block before opening
a new one, which its printed run never exercises.

Swapping ("KV-Cache Management and PagedAttention", section "What paging unlocks downstream",
preemption and eviction; "PagedAttention and KV Cache Management", section "Continuous Batching vs.
Static Batching", preemption and GPU swapping): the block manager may preempt sequences by moving
their blocks to host memory and later bring them back. The pages give no procedure, so the model
takes the plainest reading that keeps the per-block accounting of the rules above:

* a group of sequences is swapped together; every distinct block of the group's tables gets one
  block on the other side (taken from that side's free list, front first, in order of first
  appearance: sequences in the given order, each table in logical order), so blocks shared
  inside the group stay shared with the same reference counts;
* each table entry then drops one reference on its old block (blocks at zero go to the back of
  their free list, in that same order) and points at the new block;
* a swapped-out sequence cannot be appended to or forked; releasing it frees its host blocks;
* like every other operation, a swap either succeeds completely or changes nothing.

The model tracks token counts, not token ids: the K and V rows themselves live in the device pool.
A decode step asks it for the slot of each new token (``slot = block * B + offset``) and for the
block copies copy-on-write needs.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple


class OutOfBlocks(MemoryError):
    """The free list cannot supply the blocks an operation needs (nothing was changed)."""


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int, num_host_blocks: int = 0):
        if num_blocks <= 0 or block_size <= 0 or num_host_blocks < 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free: List[int] = list(range(num_blocks))    # popped from the front
        self.ref: List[int] = [0] * num_blocks
        self.host_free: List[int] = list(range(num_host_blocks))
        self.host_ref: List[int] = [0] * num_host_blocks
        self.tables: Dict[int, List[int]] = {}
        self.tokens: Dict[int, int] = {}
        self.on_host: set = set()      # swapped-out sequences (their tables hold host blocks)

    # -- queries ---------------------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def num_free_host(self) -> int:
        return len(self.host_free)

    def is_swapped(self, seq: int) -> bool:
        return seq in self.on_host

    def table(self, seq: int) -> List[int]:
        return list(self.tables[seq])

    def num_tokens(self, seq: int) -> int:
        return self.tokens[seq]

    # -- helpers ---------------------------------------------------------------------------
    def _pop(self) -> int:
        if not self.free:
            raise OutOfBlocks("no free physical blocks")
        b = self.free.pop(0)
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    # -- operations ------------------------------------------------------------------------
    def allocate(self, seq: int, num_tokens: int) -> List[int]:
        """A new sequence with a prompt of num_tokens: ceil(num_tokens / B) fresh blocks."""
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        need = -(-num_tokens // self.block_size)
        if need > len(self.free):
            raise OutOfBlocks(f"{need} blocks needed, {len(self.free)} free")
        self.tables[seq] = [self._pop() for _ in range(need)]
        self.tokens[seq] = num_tokens
        return self.table(seq)

    def append(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """One new token at the end of seq. Returns (slot, copy) where copy is the (src, dst) block
        copy that copy-on-write needs before the token is written, or None."""
        if seq in self.on_host:
            raise KeyError(f"sequence {seq} is swapped out")
        table = self.tables[seq]
        pos = self.tokens[seq]
        copy = None
        if pos % self.block_size == 0:
            # boundary: the token opens a new logical block
            table.append(self._pop())
        else:
            last = table[pos // self.block_size]
            if self.ref[last] > 1:
                # the token would modify a block other sequences still read: copy it first
                fresh = self._pop()
                self.ref[last] -= 1
                table[pos // self.block_size] = fresh
                copy = (last, fresh)
        self.tokens[seq] = pos + 1
        slot = table[pos // self.block_size] * self.block_size + pos % self.block_size
        return slot, copy

    def append_batch(self, seqs: List[int]) -> Tuple[List[int], List[Tuple[int, int]]]:
        """append() for each listed sequence in order; all or nothing on OutOfBlocks."""
        saved = (list(self.free), list(self.ref), {s: list(t) for s, t in self.tables.items()},
                 dict(self.tokens))
        slots, copies = [], []
        try:
            for s in seqs:
                slot, copy = self.append(s)
                slots.append(slot)
                if copy is not None:
                    copies.append(copy)
        except OutOfBlocks:
            self.free, self.ref, self.tables, self.tokens = saved
            raise
        return slots, copies

    def fork(self, src: int, dst: int) -> List[int]:
        """dst shares every block of src (reference counts + 1); nothing is copied."""
        if dst in self.tables:
            raise KeyError(f"sequence {dst} exists")
        if src in self.on_host:
            raise KeyError(f"sequence {src} is swapped out")
        for b in self.tables[src]:
            self.ref[b] += 1
        self.tables[dst] = list(self.tables[src])
        self.tokens[dst] = self.tokens[src]
        return self.table(dst)

    def release(self, seq: int) -> None:
        """The sequence ends: every block loses one reference; blocks at zero return to the back
        of the free list, in table order."""
        table = self.tables.pop(seq)
        del self.tokens[seq]
        if seq in self.on_host:
            self.on_host.discard(seq)
            for h in table:
                self.host_ref[h] -= 1
                if self.host_ref[h] == 0:
                    self.host_free.append(h)
            return
        for b in table:
            self._release(b)

    # -- swapping ----------------------------------------------------------------------------
    def _move(self, seqs: List[int], to_host: bool) -> List[Tuple[int, int]]:
        if len(set(seqs)) != len(seqs):
            raise KeyError("a sequence is listed twice")
        for s in seqs:
            if s not in self.tables:
                raise KeyError(f"sequence {s}")
            if (s in self.on_host) == to_host:
                raise KeyError(f"sequence {s} is already {'on the host' if to_host else 'on the device'}")
        src_ref = self.ref if to_host else self.host_ref
        dst_ref = self.host_ref if to_host else self.ref
        src_free = self.free if to_host else self.host_free
        dst_free = self.host_free if to_host else self.free
        order: List[int] = []            # distinct blocks in order of first appearance
        seen = set()
        for s in seqs:
            for b in self.tables[s]:
                if b not in seen:
                    seen.add(b)
                    order.append(b)
        if len(order) > len(dst_free):
            raise OutOfBlocks(f"{len(order)} blocks needed, {len(dst_free)} free")
        mapping = {}
        for b in order:
            nb = dst_free.pop(0)
            dst_ref[nb] = 0
            mapping[b] = nb
        for s in seqs:
            t = self.tables[s]
            for j, b in enumerate(t):
                dst_ref[mapping[b]] += 1
                src_ref[b] -= 1
                if src_ref[b] == 0:
                    src_free.append(b)
                t[j] = mapping[b]
            if to_host:
                self.on_host.add(s)
            else:
                self.on_host.discard(s)
        return [(b, mapping[b]) for b in order]

    def swap_out(self, seqs: List[int]) -> List[Tuple[int, int]]:
        """Preempt the group: returns the (device block, host block) copies to run before the
        device blocks are reused."""
        return self._move(list(seqs), True)

    def swap_in(self, seqs: List[int]) -> List[Tuple[int, int]]:
        """Resume the group: returns the (host block, device block) copies to run before decode."""
        return self._move(list(seqs), False)
