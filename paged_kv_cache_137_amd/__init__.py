"""Paged KV-cache attention for AMD MI355X (gfx950).

The hot path of PagedAttention.  Keys and values live in fixed-size blocks of a
shared physical pool, and each sequence finds its blocks through a block table.
Hand-written HIP kernels (libpkv.so, C ABI in include/pkv.h) do three things:
write new tokens into their slots, run decode attention block by block (with
a split-context reduce), and run causal prefill attention on the matrix cores.

    from paged_kv_cache_137_amd import PagedKVCache, paged_attn_decode, paged_attn_prefill
"""

from .blocks import BlockManager, OutOfBlocks, slot_mapping  # noqa: F401


def __getattr__(name):
    # The GPU entry points import torch and load libpkv.so on first use.
    if name in ("kv_cache_write", "paged_attn_decode", "paged_attn_decode_partial", "paged_attn_decode_reduce",
                "paged_attn_decode_shared", "decode_shared_workspace_bytes",
                "paged_attn_prefill", "paged_attn_prefill_cached", "decode_workspace_bytes", "copy_blocks",
                "swap_blocks"):
        from . import ops

        return getattr(ops, name)
    if name == "PagedKVCache":
        from .cache import PagedKVCache

        return PagedKVCache
    raise AttributeError(name)
