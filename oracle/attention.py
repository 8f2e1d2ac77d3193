"""Paged cache write, paged decode attention and causal prefill, in float64.

TEST INFRASTRUCTURE ONLY: the oracle, never the product path.

What is computed is plain softmax attention: the attention equation of "vLLM &
PagedAttention: Efficient Memory Management for LLM Serving", section I,
    a_ij = exp(q_i . k_j / sqrt(d)) / sum_{t <= i} exp(q_i . k_t / sqrt(d)),
    o_i  = sum_{j <= i} a_ij v_j.
"PagedAttention and vLLM, annotated", section 4.1, says the paged,
block-by-block evaluation gives exactly this value.  It is the same as attending
over one contiguous array.  So the oracle first reassembles each sequence's
contiguous K and V from its block list (the block-wise equation and the
logical/physical blocks of "vLLM & PagedAttention", section III).  Slots at or
past the context length are dropped: the partly filled last block of section
4.1 of the annotated page.  Then it applies the equation above, with no
blocking, tiling or online rescaling.

Layouts (the same as the GPU path's, because both read the same input bytes):
    cache  [num_blocks][num_heads][block_size][head_dim]
    q/k/v  [tokens][num_heads][head_dim]
bf16 data arrives as uint16 bit patterns.
"""

from __future__ import annotations

import numpy as np

_UINT = {2: np.uint16, 4: np.uint32, 8: np.uint64}


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements (bf16: the 16 bits are the top of a float32)."""
    if dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype in ("f16", "f32"):
        return np.asarray(x).astype(np.float64)
    raise ValueError(dtype)


def cache_write(k_cache, v_cache, k, v, slot_mapping, block_size: int):
    """Copy each new token's key and value into its slot.  Returns new pool arrays.

    For every token t with slot_mapping[t] >= 0, and every head h:
        cache[slot // B][h][slot % B][:] = new[t][h][:]
    The copy is byte-for-byte, with no conversion.  Every other byte of the pool is
    unchanged.  A negative slot marks a padding token and is skipped.
    "vLLM & PagedAttention", section X, describes this step as a fused reshape-and-block-write of the new KV into the
    block-table positions.  Section V of the same page gives the order: prompt
    tokens fill logical blocks left to right, and a decode token goes to the next
    free slot.
    """
    kc, vc = k_cache.copy(), v_cache.copy()
    ut = _UINT[kc.dtype.itemsize]
    kcu, vcu = kc.view(ut), vc.view(ut)
    ku, vu = np.asarray(k).view(ut), np.asarray(v).view(ut)
    capacity = kc.shape[0] * block_size
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        if slot >= capacity:
            raise IndexError(f"slot {slot} outside a pool of {capacity} slots")
        b, o = divmod(int(slot), block_size)
        kcu[b, :, o, :] = ku[t]
        vcu[b, :, o, :] = vu[t]
    return kc, vc


def copy_blocks(k_cache, v_cache, block_pairs):
    """Copy whole physical blocks (all heads, keys and values).  Returns new pool arrays.

    For each (src, dst) pair, cache[dst] = cache[src], byte for byte.  This is the
    copy-on-write step: a write into a shared block copies the block first, and
    the writer moves to the copy ("vLLM & PagedAttention", section VII, Figure
    8).  All copies of a step are batched into one launch (section X of the same
    page).  Pairs are applied in order.
    """
    kc, vc = k_cache.copy(), v_cache.copy()
    ut = _UINT[kc.dtype.itemsize]
    kcu, vcu = kc.view(ut), vc.view(ut)
    nb = kc.shape[0]
    for src, dst in np.asarray(block_pairs, dtype=np.int64).reshape(-1, 2):
        if not (0 <= src < nb and 0 <= dst < nb):
            raise IndexError(f"block pair ({src}, {dst}) outside a pool of {nb} blocks")
        kcu[dst] = kcu[src]
        vcu[dst] = vcu[src]
    return kc, vc


def gather(cache: np.ndarray, block_table, context_len: int, block_size: int) -> np.ndarray:
    """A sequence's contiguous [num_heads][context_len][head_dim] view, built block by block.

    Logical block j lives in physical block block_table[j] ("PagedAttention and
    vLLM, annotated", section 4.2).
    Blocks are concatenated in logical order.  Rows at or past context_len are dropped.
    """
    nb = -(-context_len // block_size)
    parts = [cache[int(block_table[j])] for j in range(nb)]  # each [H][B][D]
    full = np.concatenate(parts, axis=1) if parts else cache[:0].reshape(cache.shape[1], 0, cache.shape[3])
    return full[:, :context_len, :]


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) weighted sum of V's rows, float64.  q [D], K and V [n][D]."""
    z = scale * (K @ q)
    z = z - z.max()  # only for range; it cancels in the ratio
    p = np.exp(z)
    return (p @ V) / p.sum()


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, dtype: str,
                 block_size: int = 16, seqs=None) -> np.ndarray:
    """Decode attention for each sequence's current token; float64 [S][H][D].

    context_lens[s] includes the current token, whose key and value are already in
    the cache.  Its query attends to positions 0 .. context_lens[s]-1: the equation's
    i is the last position.  `seqs` restricts the work to some sequences.  Rows of
    the others stay NaN.
    """
    S, H, D = q.shape
    out = np.full((S, H, D), np.nan)
    for s in (range(S) if seqs is None else seqs):
        n = int(context_lens[s])
        K = to_f64(gather(k_cache, block_tables[s], n, block_size), dtype)
        V = to_f64(gather(v_cache, block_tables[s], n, block_size), dtype)
        qs = to_f64(q[s], dtype)
        for h in range(H):
            out[s, h] = attend(qs[h], K[h], V[h], scale)
    return out


def causal_prefill(q, k, v, prompt_lens, scale: float, dtype: str, prompts=None) -> np.ndarray:
    """Causal self-attention of each packed prompt; float64 [T][H][D].

    Row i of a prompt attends to rows 0..i of the same prompt: the t <= i limit of
    the attention equation in "vLLM & PagedAttention", section I.  The prompt
    phase computes all positions at once.  `prompts` restricts the work to some prompts.  Rows of the others stay NaN.
    """
    T, H, D = q.shape
    out = np.full((T, H, D), np.nan)
    offs = np.concatenate([[0], np.cumsum(np.asarray(prompt_lens, dtype=np.int64))])
    for p in (range(len(prompt_lens)) if prompts is None else prompts):
        a, b = int(offs[p]), int(offs[p + 1])
        L = b - a
        if L == 0:
            continue
        Q = to_f64(q[a:b], dtype)
        K = to_f64(k[a:b], dtype)
        V = to_f64(v[a:b], dtype)
        future = np.triu(np.ones((L, L), dtype=bool), k=1)  # j > i
        for h in range(H):
            z = scale * (Q[:, h, :] @ K[:, h, :].T)
            z[future] = -np.inf
            z = z - z.max(axis=1, keepdims=True)
            p_ = np.exp(z)
            out[a:b, h, :] = (p_ @ V[:, h, :]) / p_.sum(axis=1, keepdims=True)
    return out


def prefix_prefill(q, k_cache, v_cache, block_tables, prefix_lens, prompt_lens, scale: float, dtype: str,
                   block_size: int = 16, prompts=None) -> np.ndarray:
    """Prompt-phase attention of new tokens over a cached prefix plus themselves; float64 [T][H][D].

    Prompt p already has prefix_lens[p] tokens in the pool (the cached shared
    prefix of "vLLM & PagedAttention", section VII), followed by its
    prompt_lens[p] new tokens, whose
    K/V are in the pool too.  All of them are read through the prompt's block
    table.  New token i sits at position prefix_lens[p] + i.  It attends to
    positions 0 .. prefix_lens[p] + i, the t <= i limit of the equation in
    section I of the same page.  Compute runs only over the new tokens.  q and the output hold the
    new tokens only, packed prompt after prompt.
    """
    T, H, D = q.shape
    out = np.full((T, H, D), np.nan)
    offs = np.concatenate([[0], np.cumsum(np.asarray(prompt_lens, dtype=np.int64))])
    for p in (range(len(prompt_lens)) if prompts is None else prompts):
        C, L = int(prefix_lens[p]), int(prompt_lens[p])
        if L == 0:
            continue
        K = to_f64(gather(k_cache, block_tables[p], C + L, block_size), dtype)
        V = to_f64(gather(v_cache, block_tables[p], C + L, block_size), dtype)
        Q = to_f64(q[offs[p] : offs[p + 1]], dtype)
        for i in range(L):
            n = C + i + 1
            for h in range(H):
                out[offs[p] + i, h] = attend(Q[i, h], K[h, :n], V[h, :n], scale)
    return out
