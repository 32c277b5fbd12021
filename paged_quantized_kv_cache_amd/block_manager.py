"""Host-side block manager for the paged KV pool.

Implements the bookkeeping the pages describe for a paged cache ("KV Cache
优化实战", s2.2 and s4.4): fixed-size physical blocks, a per-sequence block
table mapping logical block i to a physical id, a new block only when a
sequence outgrows its last one, prefix sharing by pointing several tables at
the same physical blocks (reference counted), and copy-on-write when a
sequence must write into a block that others still share.

Physical ids come from a shuffled free list, so consecutive logical blocks
land anywhere in the pool.  The manager never touches device memory: it
returns slots for ``kvq_cache_write`` and (src, dst) block pairs for
``kvq_copy_blocks``.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np

TABLE_PAD = -1  # value of table entries past a sequence's last block
SHARED_HINT = 1 << 30  # table-entry bit: block read by several sequences


class PoolExhausted(RuntimeError):
    """Raised when no free block is left (a serving layer would queue)."""


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
        self._blocks: Dict[int, List[int]] = {}
        self._len: Dict[int, int] = {}

    # ------------------------------------------------------------ sequences
    def add_sequence(self, seq: int) -> None:
        if seq in self._blocks:
            raise KeyError("sequence %d exists" % seq)
        self._blocks[seq] = []
        self._len[seq] = 0

    def drop_sequence(self, seq: int) -> None:
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
