"""Host-side block manager for the paged KV pool.

Implements the bookkeeping the pages describe for a paged cache ("KV Cache
优化实战", s2.2 and s4.4): fixed-size physical blocks, a per-sequence block
table mapping logical block i to a physical id, a new block only when a
sequence outgrows its last one, prefix sharing by pointing several tables at
the same physical blocks (reference counted), and copy-on-write when a
sequence must write into a block that others still share.

Physical ids come from a shuffled free list, so consecutive logical blocks
land anywhere in the pool.  The manager never touches device memory: it
returns slots for ``kvq_cache_write``, (src, dst) block pairs for
``kvq_copy_blocks`` and (block, swap slot) pairs for ``kvq_swap_out`` /
``kvq_swap_in``.

Eviction and preemption (xpshop.cn article 402, s3: blocks are evicted by
block-level LRU, so a long session's early context is not lost to its own
tail; article 312, s3 and s6: under memory pressure a low-priority request
is preempted, its KV swapped out and brought back later): every block keeps
the step it was last read at (``touch``), ``preempt`` picks victims by
priority and then by least recent use, and ``swap_out`` / ``swap_in`` move a
sequence's private blocks to host swap slots and back into freshly allocated
blocks, while the blocks it shares stay in the pool and come back shared.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np

TABLE_PAD = -1  # value of table entries past a sequence's last block
SHARED_HINT = 1 << 30  # table-entry bit: block read by several sequences


class PoolExhausted(RuntimeError):
    """Raised when no free block is left (a serving layer would queue)."""


class SwapSpace:
    """Host-side free list of swap slots (one block each)."""

    def __init__(self, num_slots: int):
        self.num_slots = num_slots
        self._free: List[int] = list(range(num_slots))[::-1]

    def alloc(self, n: int) -> List[int]:
        if n > len(self._free):
            raise PoolExhausted("no free swap slot")
        return [self._free.pop() for _ in range(n)]

    def release(self, slots: List[int]) -> None:
        self._free.extend(slots)

    def num_free(self) -> int:
        return len(self._free)


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int,
                 rng: Optional[np.random.Generator] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        order = np.arange(num_blocks)
        if rng is not None:
            order = rng.permutation(num_blocks)
        self._free: List[int] = [int(x) for x in order[::-1]]  # pop() = order[0]
        self.refcount = np.zeros(num_blocks, np.int32)
        self.last_use = np.zeros(num_blocks, np.int64)  # step of the last read
        self._clock = 0
        self._blocks: Dict[int, List[int]] = {}
        self._len: Dict[int, int] = {}
        # swapped-out sequences: per logical block, (kept shared block, -1)
        # or (-1, swap slot)
        self._swapped: Dict[int, List[Tuple[int, int]]] = {}

    # ------------------------------------------------------------ sequences
    def add_sequence(self, seq: int) -> None:
        if seq in self._blocks:
            raise KeyError("sequence %d exists" % seq)
        self._blocks[seq] = []
        self._len[seq] = 0

    def drop_sequence(self, seq: int, space: Optional[SwapSpace] = None) -> None:
        if seq in self._swapped:
            entries = self._swapped.pop(seq)
            if space is not None:
                space.release([slot for kept, slot in entries if kept < 0])
            for kept, _ in entries:
                if kept >= 0:
                    self._release(kept)
        else:
            for blk in self._blocks.pop(seq):
                self._release(blk)
        del self._len[seq]

    def fork(self, parent: int, child: int) -> None:
        """``child`` shares every block of ``parent`` (prefix sharing)."""
        if child in self._blocks:
            raise KeyError("sequence %d exists" % child)
        blocks = list(self._blocks[parent])
        for blk in blocks:
            self.refcount[blk] += 1
        self._blocks[child] = blocks
        self._len[child] = self._len[parent]

    def length(self, seq: int) -> int:
        return self._len[seq]

    def blocks(self, seq: int) -> List[int]:
        return list(self._blocks[seq])

    # ------------------------------------------------------------ slots
    def append_slot(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot for the next token of ``seq``.

        Returns ``(slot, copy)`` where ``slot = block * block_size + offset``
        and ``copy`` is a ``(src, dst)`` pair when the last block was shared
        and had to be copied before writing into it (copy-on-write)."""
        n = self._len[seq]
        blocks = self._blocks[seq]
        off = n % self.block_size
        copy = None
        if off == 0:
            blocks.append(self._alloc())
        else:
            last = blocks[-1]
            if self.refcount[last] > 1:
                dst = self._alloc()
                self.refcount[last] -= 1
                blocks[-1] = dst
                copy = (last, dst)
        self._len[seq] = n + 1
        return blocks[-1] * self.block_size + off, copy

    # ------------------------------------------------------------ LRU, swap
    def touch(self, seqs) -> None:
        """One decode step read every block of ``seqs``."""
        self._clock += 1
        for s in seqs:
            for blk in self._blocks[s]:
                self.last_use[blk] = self._clock

    def lru_blocks(self) -> List[int]:
        """Blocks in use, least recently read first (ties by id)."""
        used = np.nonzero(self.refcount > 0)[0]
        return [int(b) for b in used[np.lexsort((used, self.last_use[used]))]]

    def resident(self, seq: int) -> bool:
        return seq in self._blocks

    def swap_out(self, seq: int, space: SwapSpace) -> List[Tuple[int, int]]:
        """Move ``seq`` to host swap slots.  Returns the (block, slot) pairs
        to copy with ``kvq_swap_out``; those blocks are released at once, so
        the copy must be issued before anything writes into them (same
        stream order is enough).

        Blocks that other sequences still hold (a shared prefix, a fork's
        blocks) are neither copied nor released: shared blocks are never
        written in place (copy-on-write), so the swapped-out sequence keeps
        its reference and ``swap_in`` maps the same blocks again, still
        shared.  If the swap space cannot take the private blocks, nothing
        changes and PoolExhausted is raised."""
        blocks = self._blocks[seq]
        private = [b for b in blocks if self.refcount[b] == 1]
        slots = iter(space.alloc(len(private)))      # raises before any change
        del self._blocks[seq]
        entries = []                                 # (kept block or -1, slot or -1)
        pairs = []
        for blk in blocks:
            if self.refcount[blk] == 1:
                slot = next(slots)
                pairs.append((blk, slot))
                entries.append((-1, slot))
                self._release(blk)
            else:
                entries.append((blk, -1))
        self._swapped[seq] = entries
        return pairs

    def swap_in(self, seq: int, space: SwapSpace) -> List[Tuple[int, int]]:
        """Bring ``seq`` back: its private blocks into freshly allocated ones
        (the returned (block, slot) pairs, to copy with ``kvq_swap_in``; the
        slots are free again once that copy has run), its shared blocks as
        they were."""
        entries = self._swapped[seq]
        need = sum(1 for kept, _ in entries if kept < 0)
        if need > len(self._free):
            raise PoolExhausted("not enough free KV blocks to swap in")
        del self._swapped[seq]
        blocks, pairs = [], []
        for kept, slot in entries:
            if kept >= 0:
                blocks.append(kept)
            else:
                blk = self._alloc()
                blocks.append(blk)
                pairs.append((blk, slot))
        self._blocks[seq] = blocks
        space.release([slot for _, slot in pairs])
        return pairs

    def preempt(self, need_blocks: int, priority: Dict[int, int],
                space: SwapSpace) -> List[Tuple[int, List[Tuple[int, int]]]]:
        """Swap out resident sequences until ``need_blocks`` blocks are free:
        lowest priority first, then the sequence whose blocks were read least
        recently.  Returns ``[(seq, pairs)]`` in swap-out order."""
        out = []
        cands = [s for s in self._blocks if self._blocks[s]]
        cands.sort(key=lambda s: (priority.get(s, 0),
                                  int(self.last_use[self._blocks[s]].max()), s))
        for s in cands:
            if len(self._free) >= need_blocks:
                break
            out.append((s, self.swap_out(s, space)))
        if len(self._free) < need_blocks:
            raise PoolExhausted("preemption cannot free %d blocks" % need_blocks)
        return out

    # ------------------------------------------------------------ tables
    def tables(self, num_seqs: int, max_blocks: Optional[int] = None,
               mark_shared: bool = False) -> np.ndarray:
        """Block tables ``int32 [num_seqs][width]``.  With ``mark_shared``,
        entries of blocks held by more than one sequence carry SHARED_HINT
        (bit 30), the decode kernel's cache-policy hint."""
        width = max((len(self._blocks.get(s, [])) for s in range(num_seqs)),
                    default=0)
        width = max(width, 1) if max_blocks is None else max_blocks
        t = np.full((num_seqs, width), TABLE_PAD, np.int32)
        for s in range(num_seqs):
            bl = self._blocks.get(s, [])
            if len(bl) > width:
                raise ValueError("table width too small")
            ids = np.asarray(bl, np.int64)
            if mark_shared and ids.size:
                ids = np.where(self.refcount[ids] > 1, ids | SHARED_HINT, ids)
            t[s, :len(bl)] = ids
        return t

    def used_blocks(self) -> List[int]:
        return [i for i in range(self.num_blocks) if self.refcount[i] > 0]

    def num_free(self) -> int:
        return len(self._free)

    # ------------------------------------------------------------ internals
    def _alloc(self) -> int:
        if not self._free:
            raise PoolExhausted("no free KV block")
        blk = self._free.pop()
        self.refcount[blk] = 1
        return blk

    def _release(self, blk: int) -> None:
        self.refcount[blk] -= 1
        if self.refcount[blk] == 0:
            self._free.append(blk)
