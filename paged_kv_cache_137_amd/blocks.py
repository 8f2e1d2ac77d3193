"""Host-side block bookkeeping: the KV cache manager's tables, on the CPU.

The manager owns the physical block pool's free list.  For every sequence it
keeps the logical-to-physical block table ("PagedAttention and vLLM, annotated",
section 4.2) and its token count.  It also keeps a reference count per
physical block, so that sequences can share blocks.  From these it produces what
the GPU kernels consume: int32 block tables, int32 context lengths and the
int64 slot of each new token.  Slot = physical block * block_size + offset
within the block.

Behaviour follows "vLLM & PagedAttention: Efficient Memory Management for LLM
Serving":
  - section V, Figure 6: a prompt takes only the blocks it needs, filled left to
    right.  A new token goes to the free slot of the last block, and a new block
    is allocated only when that block is full.
  - section VII, Figure 8: fork shares every block and raises its count.  A write
    into a shared block copies that block first (copy-on-write), moves the
    writer to the copy and decrements the original's count.  Full shared blocks
    are never copied.
  - section X: sequences are built from fork, append and free.
Freed blocks (count 0) go back to the free list and can be reused at once.
"""

from __future__ import annotations

from collections import deque

import numpy as np


class OutOfBlocks(RuntimeError):
    """No free physical block is left."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = range(num_blocks) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the pool")
        self._free = deque(order)
        self.ref = np.zeros(num_blocks, dtype=np.int32)
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.pending_copies: list[tuple[int, int]] = []

    # -- allocation ---------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self._free)

    def _take(self) -> int:
        if not self._free:
            raise OutOfBlocks("no free KV block")
        b = self._free.popleft()
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] < 0:
            raise AssertionError(f"block {b} released more often than referenced")
        if self.ref[b] == 0:
            self._free.append(b)

    def _slot(self, table: list[int], pos: int) -> int:
        return table[pos // self.block_size] * self.block_size + pos % self.block_size

    # -- sequence primitives --------------------------------------------------
    def add_sequence(self, seq: int, num_tokens: int) -> np.ndarray:
        """A new sequence holding `num_tokens` prompt tokens; returns their slots (int64)."""
        if seq in self.tables:
            raise ValueError(f"sequence {seq} exists")
        nb = -(-num_tokens // self.block_size)
        if nb > self.num_free:
            raise OutOfBlocks(f"sequence {seq} needs {nb} blocks, {self.num_free} free")
        table = [self._take() for _ in range(nb)]
        self.tables[seq] = table
        self.lens[seq] = num_tokens
        return np.asarray([self._slot(table, p) for p in range(num_tokens)], dtype=np.int64)

    def append_token(self, seq: int) -> int:
        """Room for one more token of `seq`; returns its slot.

        When the last block is shared, it is copied first: the (source,
        destination) pair is queued in pending_copies for the device-side copy.
        A step applies take_copies() (pkv_copy_blocks) before it writes the
        step's new tokens, so every copy sees the block as it was before the step.
        """
        table = self.tables[seq]
        pos = self.lens[seq]
        if pos % self.block_size == 0:
            table.append(self._take())
        else:
            last = table[-1]
            if self.ref[last] > 1:
                fresh = self._take()
                self.pending_copies.append((last, fresh))
                self.ref[last] -= 1
                table[-1] = fresh
        self.lens[seq] = pos + 1
        return self._slot(table, pos)

    def fork(self, parent: int, child: int) -> None:
        """`child` starts as `parent`: same blocks, one more reference each."""
        if child in self.tables:
            raise ValueError(f"sequence {child} exists")
        table = list(self.tables[parent])
        for b in table:
            self.ref[b] += 1
        self.tables[child] = table
        self.lens[child] = self.lens[parent]

    def free(self, seq: int) -> None:
        for b in self.tables.pop(seq):
            self._release(b)
        del self.lens[seq]

    def take_copies(self) -> list[tuple[int, int]]:
        out, self.pending_copies = self.pending_copies, []
        return out

    # -- arrays for the kernels ----------------------------------------------
    def block_tables(self, seqs, width: int | None = None, pad: int = 0) -> np.ndarray:
        seqs = list(seqs)
        w = max([len(self.tables[s]) for s in seqs] + [1]) if width is None else width
        t = np.full((len(seqs), w), pad, dtype=np.int32)
        for i, s in enumerate(seqs):
            t[i, : len(self.tables[s])] = self.tables[s]
        return t

    def context_lens(self, seqs) -> np.ndarray:
        return np.asarray([self.lens[s] for s in seqs], dtype=np.int32)

    def filled(self, seq: int) -> list[int]:
        """The '#filled' column of the sequence's block table."""
        n, B = self.lens[seq], self.block_size
        return [min(B, n - j * B) for j in range(len(self.tables[seq]))]


def slot_mapping(block_tables: np.ndarray, seq_index, positions, block_size: int = 16) -> np.ndarray:
    """Slots of (sequence row, position) pairs under the given int32 tables; int64."""
    rows = np.asarray(seq_index, dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)
    phys = block_tables[rows, pos // block_size].astype(np.int64)
    return phys * block_size + pos % block_size
