"""Paged KV-cache attention for AMD MI355X (gfx950).

The hot path of PagedAttention: keys and values live in fixed-size blocks of a
shared physical pool, each sequence finds its blocks through a block table, and
hand-written HIP kernels write new tokens into their slots, run decode attention
block by block, and run causal prefill attention.
"""
