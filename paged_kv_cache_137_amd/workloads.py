"""Seeded synthetic inputs for the paged KV-cache attention path.

This module draws random numbers and lays them out in the shapes the path
consumes.  It computes no part of the method itself: no attention, no softmax,
no slot arithmetic.  The GPU tests, the benchmark and the CPU oracle all take
their inputs from here, so the two sides of every parity check see the very same
bytes.

Shapes follow the models the pages discuss: the OPT-13B head shape (40 heads of
128) and a Llama-2-7B head shape (32 x 128), with 16-token blocks, the default
block size ("PagedAttention and vLLM, annotated", section 7.2; "vLLM &
PagedAttention: Efficient Memory Management for LLM Serving", section V).  The
evaluation there runs ShareGPT and Alpaca request traces (same dissection,
section XI), which are not available here.  Seeded length distributions stand in
for them: uniform and lognormal, with high variance.

Values are N(0, 1), drawn in float32 and rounded to the storage type
(round-to-nearest-even).  bfloat16 is carried as raw uint16 bit patterns,
because numpy has no bfloat16 type.  Large arrays are filled in fixed chunks.
Each chunk has its own generator, keyed by (seed, stream, chunk index), so the
values do not depend on how many threads fill them.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16
DTYPES = ("f32", "f16", "bf16")
SEED_BASE = 137000

# Random streams within one seed.  Each tensor has its own stream, so adding or
# removing one tensor never shifts the values of another.
_S_KPOOL, _S_VPOOL, _S_Q, _S_KNEW, _S_VNEW, _S_QP, _S_KP, _S_VP = range(1, 9)

_CHUNK = 1 << 22


def storage_dtype(dtype: str):
    """numpy type that carries one element of `dtype` (bf16 as uint16 bits)."""
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def elem_bytes(dtype: str) -> int:
    return {"f32": 4, "f16": 2, "bf16": 2}[dtype]


def nan_value(dtype: str):
    """A quiet NaN in the storage type; used to poison slots a correct kernel never reads."""
    if dtype == "bf16":
        return np.uint16(0x7FC0)
    return storage_dtype(dtype)(np.nan)


def _threads() -> int:
    n = int(os.environ.get("PKV_GEN_THREADS", "0") or 0)
    if n <= 0:
        try:
            n = len(os.sched_getaffinity(0))
        except AttributeError:  # pragma: no cover
            n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x32
    if dtype == "f16":
        return x32.astype(np.float16)
    # bfloat16: round the float32 bit pattern to its upper 16 bits, ties to even.
    u = x32.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def normal(key: tuple, shape, dtype: str) -> np.ndarray:
    """N(0, 1) values of `shape`, rounded to `dtype` storage, from generator key `key`."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=storage_dtype(dtype))
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)

    def fill(c: int) -> None:
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        rng = np.random.default_rng(list(key) + [c])
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = _to_storage(x, dtype)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(min(_threads(), nchunks)) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


# ---------------------------------------------------------------------------
# Containers
# ---------------------------------------------------------------------------


@dataclass
class DecodeInputs:
    """One decode step over a paged pool.

    k_cache, v_cache: [num_blocks][num_heads][block_size][head_dim], storage dtype.
    block_tables:     int32 [S][max_blocks]; entries past a sequence's last block
                      hold `pad_block`, a block no sequence owns.
    context_lens:     int32 [S]; includes the current token.
    q:                [S][num_heads][head_dim]; the current token's query.
    k_new, v_new:     [S][num_heads][head_dim] or None.  When present, the current
                      token's key/value is NOT yet in the pool; the step writes it
                      (at position context_len-1) before attending.
    poisoned:         when True, every pool slot no sequence reads (including the
                      pad block and, with k_new, the current-token slots) holds NaN.
    """

    name: str
    dtype: str
    num_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    context_lens: np.ndarray
    block_tables: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    q: np.ndarray
    pad_block: int
    k_new: np.ndarray | None = None
    v_new: np.ndarray | None = None
    poisoned: bool = True
    info: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0


@dataclass
class PrefillInputs:
    """Packed variable-length prompts: q, k, v are [T][num_heads][head_dim], T = sum(prompt_lens)."""

    dtype: str
    num_heads: int
    head_dim: int
    prompt_lens: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    # Freshly allocated physical blocks that receive the prompts' K/V (int32
    # [P][max_blocks], padded with the pool's pad block); None for prefill alone.
    block_tables: np.ndarray | None = None

    @property
    def total_tokens(self) -> int:
        return int(self.prompt_lens.sum())


@dataclass
class MixedInputs:
    """One mixed step: prompts to prefill plus sequences to decode over one shared pool."""

    decode: DecodeInputs
    prefill: PrefillInputs


# ---------------------------------------------------------------------------
# Building blocks
# ---------------------------------------------------------------------------


def _blocks_for(n_tokens: np.ndarray, block_size: int) -> np.ndarray:
    # Allocation rule of the harness: a sequence is handed blocks until their
    # capacity reaches its token count.
    n = np.asarray(n_tokens, dtype=np.int64)
    return (n + block_size - 1) // block_size


def _pool_size(need: int, spare: float) -> int:
    return int(math.ceil(need * (1.0 + spare))) + 1


def _fill_tables(owned: list[np.ndarray], pad_block: int) -> np.ndarray:
    width = max([len(o) for o in owned] + [1])
    t = np.full((len(owned), width), pad_block, dtype=np.int32)
    for s, o in enumerate(owned):
        t[s, : len(o)] = o
    return t


def _poison(k_cache, v_cache, tables, present_lens, block_size, dtype) -> int:
    """NaN every slot not holding one of the first present_lens[s] tokens of some sequence.

    Returns the number of distinct slots that stay readable.
    """
    nb = k_cache.shape[0]
    used = np.zeros((nb, block_size), dtype=bool)
    for s in range(tables.shape[0]):
        n = int(present_lens[s])
        nfull, rem = divmod(n, block_size)
        if nfull:
            used[tables[s, :nfull]] = True
        if rem:
            used[tables[s, nfull], :rem] = True
    bi, oi = np.nonzero(~used)
    nan = nan_value(dtype)
    k_cache[bi, :, oi, :] = nan
    v_cache[bi, :, oi, :] = nan
    return int(used.sum())


def _lognormal_lens(rng, n, median, sigma, lo, hi) -> np.ndarray:
    x = rng.lognormal(mean=math.log(median), sigma=sigma, size=n)
    return np.clip(np.rint(x), lo, hi).astype(np.int32)


# ---------------------------------------------------------------------------
# Generic builders
# ---------------------------------------------------------------------------


def make_decode(
    seed: int,
    dtype: str,
    num_heads: int,
    head_dim: int,
    context_lens,
    *,
    block_size: int = BLOCK_SIZE,
    num_blocks: int | None = None,
    spare: float = 0.10,
    scale: float | None = None,
    poison: bool = True,
    with_new_tokens: bool = False,
    name: str = "custom",
) -> DecodeInputs:
    """A decode batch whose sequences own shuffled physical blocks of one pool.

    Draw order: physical-id permutation, q, pool K, pool V, new-token K/V.
    """
    rng = np.random.default_rng(seed)
    ctx = np.asarray(context_lens, dtype=np.int32)
    need = _blocks_for(ctx, block_size)
    total = int(need.sum())
    if num_blocks is None:
        num_blocks = _pool_size(total, spare)
    if num_blocks < total + 1:
        raise ValueError("pool too small for the batch plus a pad block")
    perm = rng.permutation(num_blocks).astype(np.int32)
    offs = np.concatenate([[0], np.cumsum(need)])
    owned = [perm[offs[s] : offs[s + 1]] for s in range(len(ctx))]
    pad = int(perm[total])
    tables = _fill_tables(owned, pad)
    S = len(ctx)
    q = normal((seed, _S_Q), (S, num_heads, head_dim), dtype)
    kc = normal((seed, _S_KPOOL), (num_blocks, num_heads, block_size, head_dim), dtype)
    vc = normal((seed, _S_VPOOL), (num_blocks, num_heads, block_size, head_dim), dtype)
    k_new = v_new = None
    present = ctx
    if with_new_tokens:
        k_new = normal((seed, _S_KNEW), (S, num_heads, head_dim), dtype)
        v_new = normal((seed, _S_VNEW), (S, num_heads, head_dim), dtype)
        present = ctx - 1
    info = {}
    if poison:
        info["readable_slots"] = _poison(kc, vc, tables, present, block_size, dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return DecodeInputs(
        name=name, dtype=dtype, num_heads=num_heads, head_dim=head_dim,
        block_size=block_size, num_blocks=num_blocks, scale=float(scale),
        context_lens=ctx, block_tables=tables, k_cache=kc, v_cache=vc, q=q,
        pad_block=pad, k_new=k_new, v_new=v_new, poisoned=poison, info=info,
    )


def make_prefill(seed: int, dtype: str, num_heads: int, head_dim: int, prompt_lens) -> PrefillInputs:
    lens = np.asarray(prompt_lens, dtype=np.int32)
    T = int(lens.sum())
    shape = (T, num_heads, head_dim)
    return PrefillInputs(
        dtype=dtype, num_heads=num_heads, head_dim=head_dim, prompt_lens=lens,
        q=normal((seed, _S_QP), shape, dtype),
        k=normal((seed, _S_KP), shape, dtype),
        v=normal((seed, _S_VP), shape, dtype),
    )


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny decode, fp32: 4 seqs, 4x64, ctx {1,17,100,300}, 64-block pool",
    2: "OPT-13B-shape decode, fp16: 64 seqs, 40x128, ctx U[1,2048]",
    3: "Llama-2-7B-shape decode, bf16: 256 seqs, 32x128, ctx lognormal(600,0.8) in [16,4096]",
    4: "block-sharing decode, fp16: 40x128, 128 prompts x 4 samples, CoW partial block",
    5: "mixed step, bf16: 32x128, 8 prompts U[128,2048] prefill + 192 decodes lognormal(800,0.8)",
}


def config_seed(index: int) -> int:
    return SEED_BASE + index


def decode_config(index: int, *, poison: bool = True, with_new_tokens: bool = False) -> DecodeInputs:
    """Configs 1-4 (decode steps)."""
    seed = config_seed(index)
    if index == 1:
        return make_decode(seed, "f32", 4, 64, [1, 17, 100, 300], num_blocks=64, scale=1.0 / 8.0,
                           poison=poison, with_new_tokens=with_new_tokens, name=CONFIG_NAMES[1])
    if index == 2:
        lens = np.random.default_rng([seed, 0]).integers(1, 2049, size=64).astype(np.int32)
        return make_decode(seed, "f16", 40, 128, lens, poison=poison,
                           with_new_tokens=with_new_tokens, name=CONFIG_NAMES[2])
    if index == 3:
        lens = _lognormal_lens(np.random.default_rng([seed, 0]), 256, 600, 0.8, 16, 4096)
        return make_decode(seed, "bf16", 32, 128, lens, poison=poison,
                           with_new_tokens=with_new_tokens, name=CONFIG_NAMES[3])
    if index == 4:
        return sharing_config(poison=poison, with_new_tokens=with_new_tokens)
    raise ValueError(f"no decode config {index}")


def sharing_config(*, groups: int = 128, samples: int = 4, poison: bool = True,
                   with_new_tokens: bool = False, seed: int | None = None,
                   prompt_range=(64, 1024), gen_range=(1, 256)) -> DecodeInputs:
    """Config 4: parallel samples share their prompt's physical blocks.

    Every group's samples reference the same physical blocks for the prompt's full
    blocks.  If the prompt ends inside a block, that partly filled block is
    copy-on-write: samples 0..n-2 each get a private copy holding the prompt's
    tokens, and the last sample keeps the original (the order of the
    parallel-sampling example in "vLLM & PagedAttention: Efficient Memory
    Management for LLM Serving", section VII, Figure 8).  Generated tokens go to
    private blocks.
    """
    B = BLOCK_SIZE
    seed = config_seed(4) if seed is None else seed
    H, D, dtype = 40, 128, "f16"
    lr = np.random.default_rng([seed, 0])
    P = lr.integers(prompt_range[0], prompt_range[1] + 1, size=groups).astype(np.int64)
    G = lr.integers(gen_range[0], gen_range[1] + 1, size=groups * samples).astype(np.int64)
    ctx = (np.repeat(P, samples) + G).astype(np.int32)

    # Count distinct physical blocks, then hand out a permutation in that order.
    n_prompt = _blocks_for(P, B)
    partial = (P % B) != 0
    plan = []  # per group: (n_prompt_blocks, partial, [per-sample new block counts])
    unique = 0
    for g in range(groups):
        own = [int(_blocks_for(ctx[g * samples + i], B) - n_prompt[g]) for i in range(samples)]
        copies = (samples - 1) if partial[g] else 0
        plan.append((int(n_prompt[g]), bool(partial[g]), own))
        unique += int(n_prompt[g]) + copies + sum(own)
    rng = np.random.default_rng(seed)
    num_blocks = _pool_size(unique, 0.10)
    perm = rng.permutation(num_blocks).astype(np.int32)
    cur = 0
    owned: list[np.ndarray] = []
    cow_pairs = []  # (original, copy) physical ids
    for g, (npb, part, own) in enumerate(plan):
        shared = perm[cur : cur + npb]
        cur += npb
        for i in range(samples):
            blocks = list(shared)
            if part and i < samples - 1:
                cp = int(perm[cur]); cur += 1
                cow_pairs.append((int(shared[-1]), cp))
                blocks[-1] = cp
            blocks.extend(perm[cur : cur + own[i]]); cur += own[i]
            owned.append(np.asarray(blocks, dtype=np.int32))
    assert cur == unique
    pad = int(perm[unique])
    tables = _fill_tables(owned, pad)
    S = groups * samples
    q = normal((seed, _S_Q), (S, H, D), dtype)
    kc = normal((seed, _S_KPOOL), (num_blocks, H, B, D), dtype)
    vc = normal((seed, _S_VPOOL), (num_blocks, H, B, D), dtype)
    # The copy carries the prompt's tokens of the original block.
    for (orig, cp), g in zip(cow_pairs, np.repeat(np.nonzero(partial)[0], samples - 1)):
        r = int(P[g] % B)
        kc[cp, :, :r, :] = kc[orig, :, :r, :]
        vc[cp, :, :r, :] = vc[orig, :, :r, :]
    k_new = v_new = None
    present = ctx
    if with_new_tokens:
        k_new = normal((seed, _S_KNEW), (S, H, D), dtype)
        v_new = normal((seed, _S_VNEW), (S, H, D), dtype)
        present = ctx - 1
    info = {
        "prompt_lens": P.astype(np.int32),
        "samples": samples,
        "physical_blocks_used": unique,
        "logical_blocks": int(_blocks_for(ctx, B).sum()),
        "cow_pairs": np.asarray(cow_pairs, dtype=np.int32).reshape(-1, 2),
    }
    if poison:
        info["readable_slots"] = _poison(kc, vc, tables, present, B, dtype)
    return DecodeInputs(
        name=CONFIG_NAMES[4], dtype=dtype, num_heads=H, head_dim=D, block_size=B,
        num_blocks=num_blocks, scale=1.0 / math.sqrt(D), context_lens=ctx,
        block_tables=tables, k_cache=kc, v_cache=vc, q=q, pad_block=pad,
        k_new=k_new, v_new=v_new, poisoned=poison, info=info,
    )


def mixed_prefill(*, seed: int | None = None, num_prompts: int = 8, prompt_range=(128, 2048), heads: int = 32,
                  head_dim: int = 128, dtype: str = "bf16") -> PrefillInputs:
    """The prompts of config 5 alone: the same lengths and values as
    mixed_config's prefill, without drawing the decode pool."""
    seed = config_seed(5) if seed is None else seed
    lr = np.random.default_rng([seed, 0])
    Lp = lr.integers(prompt_range[0], prompt_range[1] + 1, size=num_prompts).astype(np.int32)
    return make_prefill(seed, dtype, heads, head_dim, Lp)


def mixed_config(*, poison: bool = True, seed: int | None = None, num_prompts: int = 8,
                 num_decodes: int = 192, prompt_range=(128, 2048), heads: int = 32,
                 head_dim: int = 128, dtype: str = "bf16") -> MixedInputs:
    """Config 5: prompts prefill into fresh shuffled blocks while other sequences decode.

    The decode sequences' current token (position context_len-1) arrives as
    k_new/v_new and is written in the same step as the prompts' K/V; the pool
    holds their earlier tokens.  The prompts' blocks are allocated but empty.
    Decode context lengths: lognormal with median 800 and sigma 0.8, clipped to
    [16, 4096].
    """
    B = BLOCK_SIZE
    seed = config_seed(5) if seed is None else seed
    lr = np.random.default_rng([seed, 0])
    Lp = lr.integers(prompt_range[0], prompt_range[1] + 1, size=num_prompts).astype(np.int32)
    ctx = _lognormal_lens(lr, num_decodes, 800, 0.8, 16, 4096)
    need_d = _blocks_for(ctx, B)
    need_p = _blocks_for(Lp, B)
    total = int(need_d.sum() + need_p.sum())
    rng = np.random.default_rng(seed)
    num_blocks = _pool_size(total, 0.10)
    perm = rng.permutation(num_blocks).astype(np.int32)
    od = np.concatenate([[0], np.cumsum(need_d)])
    base = int(od[-1])
    op = base + np.concatenate([[0], np.cumsum(need_p)])
    pad = int(perm[total])
    dtables = _fill_tables([perm[od[s] : od[s + 1]] for s in range(num_decodes)], pad)
    ptables = _fill_tables([perm[op[p] : op[p + 1]] for p in range(num_prompts)], pad)
    q = normal((seed, _S_Q), (num_decodes, heads, head_dim), dtype)
    kc = normal((seed, _S_KPOOL), (num_blocks, heads, B, head_dim), dtype)
    vc = normal((seed, _S_VPOOL), (num_blocks, heads, B, head_dim), dtype)
    k_new = normal((seed, _S_KNEW), (num_decodes, heads, head_dim), dtype)
    v_new = normal((seed, _S_VNEW), (num_decodes, heads, head_dim), dtype)
    info = {}
    if poison:
        info["readable_slots"] = _poison(kc, vc, dtables, ctx - 1, B, dtype)
    dec = DecodeInputs(
        name=CONFIG_NAMES[5], dtype=dtype, num_heads=heads, head_dim=head_dim, block_size=B,
        num_blocks=num_blocks, scale=1.0 / math.sqrt(head_dim), context_lens=ctx,
        block_tables=dtables, k_cache=kc, v_cache=vc, q=q, pad_block=pad,
        k_new=k_new, v_new=v_new, poisoned=poison, info=info,
    )
    pre = make_prefill(seed, dtype, heads, head_dim, Lp)
    pre.block_tables = ptables
    return MixedInputs(decode=dec, prefill=pre)
