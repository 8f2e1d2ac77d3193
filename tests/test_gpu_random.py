"""Seeded random cases on the GPU against the float64 oracle.

Each case draws its own shape (dtype, head_dim, block size, heads, batch),
context or prompt lengths from a mix of edge values and random ones, a
partition size (or the library's automatic choice), and a random block layout in which some neighbouring sequences
share leading blocks.  The plain decode and the shared-prefix decode must both
match the oracle on every sequence (1e-5 for fp32 inputs, 5e-3 for 16-bit
inputs, on fp32 outputs); the cached-prefix prefill must match the oracle's
causal prefill over [prefix || prompt], and the fresh prefill the oracle's
causal prefill over ragged prompts.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_137_amd import ops
from paged_kv_cache_137_amd import workloads as W
from _dev import TOL, down, up, upload_decode, nan_out

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f16", "bf16"]
EDGE = [1, 2, 7, 8, 9, 15, 16, 17, 31, 32, 33, 255, 256, 257, 511, 512, 513, 1023, 1025]
# PKV_RANDOM_FACTOR=n runs n times as many seeds of each kind (the default run is 1).
FACTOR = max(1, int(os.environ.get("PKV_RANDOM_FACTOR", "1")))


def _random_decode(seed: int) -> tuple[W.DecodeInputs, int]:
    rng = np.random.default_rng(1000 + seed)
    dt = DTYPES[seed % 3]
    D = int(rng.choice([64, 128]))
    B = int(rng.choice([8, 16, 32]))
    H = int(rng.integers(1, 9))
    S = int(rng.integers(1, 41))
    part = int(rng.choice([0, 256, 512, 1024, ops.PARTITION_AUTO]))
    lens = [int(rng.choice(EDGE)) if rng.random() < 0.5 else int(rng.integers(1, 3001)) for _ in range(S)]
    # Block ids: windows of four sequences may share a prefix of their leading blocks.
    nxt = 0
    owned = []
    for w0 in range(0, S, 4):
        win = list(range(w0, min(S, w0 + 4)))
        shared_ids: list[int] = []
        if rng.random() < 0.6:
            nsh = int(rng.integers(1, 1 + max(1, min(lens[s] for s in win) // B)))
            shared_ids = list(range(nxt, nxt + nsh))
            nxt += nsh
        for s in win:
            full = lens[s] // B
            take = shared_ids[: min(len(shared_ids), full)] if rng.random() < 0.8 else []
            blocks = list(take)
            while len(blocks) * B < lens[s]:
                blocks.append(nxt)
                nxt += 1
            owned.append(blocks)
    num_blocks = nxt + 1
    perm = rng.permutation(num_blocks).astype(np.int32)
    owned = [perm[np.asarray(b, np.int64)] for b in owned]
    pad = int(perm[nxt])
    tables = W._fill_tables(owned, pad)
    ctx = np.asarray(lens, np.int32)
    q = W.normal((2000 + seed, 3), (S, H, D), dt)
    kc = W.normal((2000 + seed, 1), (num_blocks, H, B, D), dt)
    vc = W.normal((2000 + seed, 2), (num_blocks, H, B, D), dt)
    W._poison(kc, vc, tables, ctx, B, dt)
    d = W.DecodeInputs(name=f"random {seed}", dtype=dt, num_heads=H, head_dim=D, block_size=B,
                       num_blocks=num_blocks, scale=1.0 / math.sqrt(D), context_lens=ctx, block_tables=tables,
                       k_cache=kc, v_cache=vc, q=q, pad_block=pad, poisoned=True)
    return d, part


@pytest.mark.parametrize("seed", range(24 * FACTOR))
def test_random_decode_plain_and_shared(seed):
    d, part = _random_decode(seed)
    S = d.num_seqs
    print(f"random decode {seed}: {d.dtype} D={d.head_dim} B={d.block_size} H={d.num_heads} S={S} "
          f"part={part} max_ctx={d.max_context_len}", flush=True)
    t = upload_decode(d)
    ref = oracle.attention.paged_decode(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, d.scale, d.dtype,
                                        block_size=d.block_size, seqs=list(range(S)))
    for fn in (ops.paged_attn_decode, ops.paged_attn_decode_shared):
        out = nan_out(d.q.shape, torch.float32)
        fn(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"], d.scale, out,
           max_context_len=d.max_context_len, partition_size=part)
        got = down(out)
        assert np.isfinite(got).all()
        err = float(np.abs(got - ref).max())
        print(f"  {fn.__name__}: max|err|={err:.3e}", flush=True)
        assert err <= TOL[d.dtype]


@pytest.mark.parametrize("seed", range(16 * FACTOR))
def test_random_cached_prefix_prefill(seed):
    rng = np.random.default_rng(3000 + seed)
    dt = ["f16", "bf16"][seed % 2]
    D = int(rng.choice([64, 128]))
    B = int(rng.choice([8, 16, 32]))
    H = int(rng.integers(1, 5))
    n = int(rng.integers(1, 7))
    plens = [int(rng.choice([0, 1, 63, 64, 65, 127, 128, 129])) if rng.random() < 0.4 else int(rng.integers(1, 300))
             for _ in range(n)]
    prefs = [int(rng.choice([0, 1, 16, 100, 256])) if rng.random() < 0.5 else int(rng.integers(0, 400))
             for _ in range(n)]
    print(f"random cached prefill {seed}: {dt} D={D} B={B} H={H} plens={plens} prefixes={prefs}", flush=True)
    need = [-(-(c + L) // B) for c, L in zip(prefs, plens)]
    num_blocks = sum(need) + 1
    perm = rng.permutation(num_blocks).astype(np.int32)
    owned, at = [], 0
    for k in need:
        owned.append(perm[at: at + k])
        at += k
    # Wide enough for the longest prefix plus the longest prompt (the ABI's bound).
    width = max(max(need), -(-(max(prefs) + max(plens)) // B), 1)
    tables = np.full((n, width), int(perm[-1]), np.int32)
    for r, o in enumerate(owned):
        tables[r, : len(o)] = o
    kc = W.normal((4000 + seed, 1), (num_blocks, H, B, D), dt)
    vc = W.normal((4000 + seed, 2), (num_blocks, H, B, D), dt)
    T = sum(plens)
    qn = W.normal((4000 + seed, 3), (max(T, 1), H, D), dt)[:T]
    out = nan_out((T, H, D), torch.float32)
    ops.paged_attn_prefill_cached(up(qn, dt), up(kc, dt), up(vc, dt), up(tables), up(np.asarray(prefs, np.int32)),
                                  up(np.asarray(plens, np.int32)), out, max_prompt_len=max(plens),
                                  max_prefix_len=max(prefs))
    if T == 0:
        return
    ref = oracle.attention.prefix_prefill(qn, kc, vc, tables, prefs, plens, 1 / math.sqrt(D), dt, block_size=B)
    got = down(out)
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    print(f"  max|err|={err:.3e}", flush=True)
    assert err <= TOL[dt]


@pytest.mark.parametrize("seed", range(8 * FACTOR))
def test_random_prefill(seed):
    rng = np.random.default_rng(5000 + seed)
    dt = ["f16", "bf16"][seed % 2]
    D = int(rng.choice([64, 128]))
    H = int(rng.integers(1, 5))
    n = int(rng.integers(1, 9))
    lens = [int(rng.choice([0, 1, 127, 128, 129, 255, 256, 257])) if rng.random() < 0.4 else int(rng.integers(1, 700))
            for _ in range(n)]
    print(f"random prefill {seed}: {dt} D={D} H={H} lens={lens}", flush=True)
    if sum(lens) == 0:
        lens[0] = 1
    p = W.make_prefill(6000 + seed, dt, H, D, lens)
    out = nan_out(p.q.shape, torch.float32)
    ops.paged_attn_prefill(up(p.q, dt), up(p.k, dt), up(p.v, dt), None, up(p.prompt_lens), out,
                           max_prompt_len=int(p.prompt_lens.max()))
    ref = oracle.attention.causal_prefill(p.q, p.k, p.v, p.prompt_lens, 1 / math.sqrt(D), dt)
    got = down(out)
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    print(f"  max|err|={err:.3e}", flush=True)
    assert err <= TOL[dt]
