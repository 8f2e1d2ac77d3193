"""Integer bookkeeping of a paged KV cache, written from the pages' definitions.

TEST INFRASTRUCTURE ONLY: the oracle, never the product path.

Positions are 0-based here.  The pages count tokens from 1, so token i in
section 4.1 of "PagedAttention and vLLM, annotated" is position i-1.  A slot is
numbered physical_block * block_size + offset.  The pages never number slots.
This numbering is a reading, and it is the one the cache layout
[block][head][offset][dim] realises.
"""

from __future__ import annotations

import numpy as np


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Blocks a sequence of `num_tokens` occupies: ceil(num_tokens / block_size).

    "PagedAttention and vLLM, annotated", section 4.1, worked example (the query
    at token 40 with 16-token blocks visits 3 blocks).  Section 3 of the same
    page gives 300 tokens -> 19 blocks.
    """
    if num_tokens < 0 or block_size <= 0:
        raise ValueError("bad sizes")
    return -(-num_tokens // block_size)


def wasted_slots(num_tokens: int, block_size: int) -> int:
    """Empty slots in the last, partly filled block.  Always fewer than one block.

    "PagedAttention and vLLM, annotated": section 3, tiny example (300 tokens
    waste 4 slots), and section 4.2 (the waste stays within one block);
    "vLLM & PagedAttention", section III.
    """
    return blocks_needed(num_tokens, block_size) * block_size - num_tokens


def block_token_ranges(i: int, block_size: int) -> list[tuple[int, int]]:
    """For the query at token i (1-based), each block that holds one of tokens
    1 .. i, as the first and last of those tokens it holds, in block order.

    Token t sits in logical block (t - 1) // block_size.  Each token is placed
    in its block and each block keeps the smallest and largest token it got.
    "PagedAttention and vLLM, annotated", section 4.1: token 40 with 16-token
    blocks visits (1, 16), (17, 32) and (33, 40).
    """
    if i < 0 or block_size <= 0:
        raise ValueError("bad sizes")
    held: dict[int, tuple[int, int]] = {}
    for t in range(1, i + 1):
        blk = (t - 1) // block_size
        lo, hi = held.get(blk, (t, t))
        held[blk] = (min(lo, t), max(hi, t))
    return [held[b] for b in sorted(held)]


def filled_counts(num_tokens: int, block_size: int) -> list[int]:
    """The '#filled' column of a block table: slots in use in each logical block.

    "PagedAttention and vLLM, annotated", section 4.2 figure;
    "vLLM & PagedAttention", section V, Figure 6.
    """
    return [min(block_size, num_tokens - j * block_size) for j in range(blocks_needed(num_tokens, block_size))]


def slot_of(block_table, position: int, block_size: int) -> int:
    """Physical slot of 0-based `position` in a sequence with this block table.

    Logical block position // block_size is looked up in the table: the
    logical-to-physical map of "PagedAttention and vLLM, annotated", section
    4.2, and of "vLLM & PagedAttention", section III.  The offset inside the
    block is position % block_size.
    """
    logical = position // block_size
    offset = position % block_size
    return int(block_table[logical]) * block_size + offset


def slot_mapping(block_tables, seq_ids, positions, block_size: int) -> np.ndarray:
    """Destination slot of each new token, as int64: one slot_of per (sequence, position)."""
    out = np.empty(len(positions), dtype=np.int64)
    for t, (s, p) in enumerate(zip(seq_ids, positions)):
        out[t] = slot_of(block_tables[s], int(p), block_size)
    return out


def kv_bytes_per_token(hidden: int, layers: int, bytes_per_value: int) -> int:
    """One key and one value, each `hidden` wide, per layer: 2 * h * L * b.

    "PagedAttention and vLLM, annotated", section 1, and "vLLM & PagedAttention",
    section I: OPT-13B gives 2 * 5120 * 40 * 2 = 819,200 B.
    """
    return 2 * hidden * layers * bytes_per_value


def max_kv_slots(kv_memory_bytes: float, per_token_bytes: int) -> float:
    """How many tokens' KV fit in a memory budget.

    "PagedAttention and vLLM, annotated", section 6 table (12 GB / 800 KB = 15.7K).
    """
    return kv_memory_bytes / per_token_bytes


def reservation_waste(used_tokens: int, reserved_tokens: int) -> tuple[int, float]:
    """Slots left empty by a contiguous max-length reservation, and their share of it.

    "PagedAttention and vLLM, annotated", section 3, tiny example: 300 used of
    2,048 reserved -> 1,748 wasted (85%).
    """
    w = reserved_tokens - used_tokens
    return w, w / reserved_tokens
