"""PagedKVCache: one layer's physical K/V block pool in device memory.

The pool is carved once into fixed-size blocks ("vLLM & PagedAttention:
Efficient Memory Management for LLM Serving", section III: physical KV blocks).
Its layout is [num_blocks][num_heads][block_size][head_dim] for keys and for
values.  Any free block can serve any sequence.
"""

from __future__ import annotations

import torch

from . import ops


class PagedKVCache:
    def __init__(self, num_blocks: int, num_heads: int, head_dim: int, block_size: int = 16,
                 dtype: torch.dtype = torch.bfloat16, device="cuda"):
        if block_size not in ops.BLOCK_SIZES:
            raise ValueError(f"block_size must be one of {ops.BLOCK_SIZES}")
        shape = (num_blocks, num_heads, block_size, head_dim)
        self.k_cache = torch.empty(shape, dtype=dtype, device=device)
        self.v_cache = torch.empty(shape, dtype=dtype, device=device)

    @classmethod
    def pinned_host(cls, num_blocks: int, num_heads: int, head_dim: int, block_size: int = 16,
                    dtype: torch.dtype = torch.bfloat16) -> "PagedKVCache":
        """A pool of the same layout in pinned host memory, the target of swap_out."""
        shape = (num_blocks, num_heads, block_size, head_dim)
        return cls.from_tensors(torch.empty(shape, dtype=dtype, pin_memory=True),
                                torch.empty(shape, dtype=dtype, pin_memory=True))

    @classmethod
    def from_tensors(cls, k_cache: torch.Tensor, v_cache: torch.Tensor) -> "PagedKVCache":
        self = cls.__new__(cls)
        self.k_cache, self.v_cache = k_cache, v_cache
        return self

    @property
    def num_blocks(self) -> int:
        return self.k_cache.shape[0]

    @property
    def num_heads(self) -> int:
        return self.k_cache.shape[1]

    @property
    def block_size(self) -> int:
        return self.k_cache.shape[2]

    @property
    def head_dim(self) -> int:
        return self.k_cache.shape[3]

    def kv_cache_write(self, k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor) -> None:
        """Write new tokens' keys and values into the physical blocks."""
        ops.kv_cache_write(k, v, slot_mapping, self.k_cache, self.v_cache)

    def copy_blocks(self, block_pairs: torch.Tensor) -> None:
        """Copy-on-write: copy whole blocks, (src, dst) pairs, keys and values, in one launch."""
        ops.copy_blocks(self.k_cache, self.v_cache, block_pairs)

    def paged_attn_decode(self, q, block_tables, context_lens, scale, out, **kw):
        return ops.paged_attn_decode(q, self.k_cache, self.v_cache, block_tables, context_lens, scale, out, **kw)

    def paged_attn_decode_shared(self, q, block_tables, context_lens, scale, out, **kw):
        """paged_attn_decode that reads blocks shared by neighbouring sequences once."""
        return ops.paged_attn_decode_shared(q, self.k_cache, self.v_cache, block_tables, context_lens, scale, out,
                                            **kw)

    def paged_attn_prefill_cached(self, q, block_tables, prefix_lens, prompt_lens, out, **kw):
        """Prompt phase of new tokens over cached prefixes, everything read through the tables."""
        return ops.paged_attn_prefill_cached(q, self.k_cache, self.v_cache, block_tables, prefix_lens, prompt_lens,
                                             out, **kw)

    def swap_out(self, host: "PagedKVCache", block_pairs: torch.Tensor) -> None:
        """Copy (device block, host block) pairs from this pool into a pinned host pool."""
        ops.swap_blocks(self.k_cache, self.v_cache, host.k_cache, host.v_cache, block_pairs)

    def swap_in(self, host: "PagedKVCache", block_pairs: torch.Tensor) -> None:
        """Copy (host block, device block) pairs from a pinned host pool into this pool."""
        ops.swap_blocks(host.k_cache, host.v_cache, self.k_cache, self.v_cache, block_pairs)
