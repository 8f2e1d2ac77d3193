"""Causal prefill on the GPU (MFMA) against the float64 oracle; the mixed step of config 5."""

import math

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_137_amd import ops
from paged_kv_cache_137_amd import workloads as W
from paged_kv_cache_137_amd.blocks import slot_mapping
from _dev import TOL, TORCH_DT, bits, down, nan_out, rne_to, run_decode, timed, up, upload_decode
from _records import record

pytestmark = pytest.mark.gpu


def _prefill(p, out_dtype="f32", heads=None):
    q, k, v = p.q, p.k, p.v
    if heads is not None:
        q, k, v = (np.ascontiguousarray(x[:, heads]) for x in (q, k, v))
    out = nan_out(q.shape, out_dtype)
    ops.paged_attn_prefill(up(q, p.dtype), up(k, p.dtype), up(v, p.dtype), None, up(p.prompt_lens), out,
                           max_prompt_len=int(p.prompt_lens.max()))
    return out


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("f16", 128), ("bf16", 64), ("f16", 64)])
def test_prefill_parity_ragged(dt, D):
    lens = [1, 2, 17, 63, 64, 65, 127, 128, 129, 300, 0, 513]
    print(f"prefill parity {dt} D={D}", flush=True)
    p = W.make_prefill(71, dt, 4, D, lens)
    out32 = down(_prefill(p))
    ref = oracle.attention.causal_prefill(p.q, p.k, p.v, p.prompt_lens, 1 / math.sqrt(D), dt)
    assert np.isfinite(out32).all()
    err = float(np.abs(out32 - ref).max())
    print(f"  max|err|={err:.3e}", flush=True)
    assert err <= TOL[dt]
    outdt = down(_prefill(p, dt))
    assert np.array_equal(bits(outdt), bits(rne_to(out32, dt)))
    # row 0 of every prompt is v_0 exactly
    offs = np.concatenate([[0], np.cumsum(lens)])[:-1]
    for o, L in zip(offs, lens):
        if L:
            assert np.array_equal(out32[o].astype(np.float64), oracle.attention.to_f64(p.v[o], dt))


def test_prefill_32768_token_prompt():
    """One 32,768-token prompt beside a 5-token one, 2 heads x 128, bf16: the
    longest query tile runs 1,024 key tiles.  Sampled rows (the first and last
    48 of the long prompt, 96 more at random, and every row of the short one)
    against the oracle's attention over the row's causal prefix; every output
    written; the 16-bit output is the rounding of the f32 one."""
    lens = [32768, 5]
    print("prefill, 32,768-token prompt", flush=True)
    p = W.make_prefill(83, "bf16", 2, 128, lens)
    out32 = down(_prefill(p))
    assert np.isfinite(out32).all()
    q, k, v = (oracle.attention.to_f64(x, "bf16") for x in (p.q, p.k, p.v))
    rng = np.random.default_rng(84)
    rows = sorted(set(range(48)) | set(range(32768 - 48, 32768)) | set(rng.integers(48, 32768 - 48, 96).tolist()))
    rows += [32768 + i for i in range(5)]
    err = 0.0
    for i in rows:
        start = 0 if i < 32768 else 32768
        for h in range(2):
            ref = oracle.attention.attend(q[i, h], k[start:i + 1, h], v[start:i + 1, h], 1 / math.sqrt(128))
            err = max(err, float(np.abs(out32[i, h] - ref).max()))
    print(f"  rows={len(rows)} max|err|={err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    outdt = down(_prefill(p, "bf16"))
    assert np.array_equal(bits(outdt), bits(rne_to(out32, "bf16")))


@pytest.mark.parametrize("n", [63, 64, 65])
def test_prefill_many_prompts_dense_and_sparse_enumeration(n):
    """Up to 64 prompts the kernel enumerates only existing query tiles, ranked
    by length (ties by index); above that every prompt gets the longest
    prompt's tile count.  Both sides of the boundary, with empty prompts, equal
    lengths and tile-multiple lengths, against the oracle."""
    rng = np.random.default_rng(80 + n)
    lens = [int(rng.choice([0, 1, 128, 129, 130, 255, 256])) if i % 3 else int(rng.integers(1, 400)) for i in range(n)]
    print(f"prefill {n} prompts, total {sum(lens)}", flush=True)
    p = W.make_prefill(81, "bf16", 2, 64, lens)
    out32 = down(_prefill(p))
    ref = oracle.attention.causal_prefill(p.q, p.k, p.v, p.prompt_lens, 1 / math.sqrt(64), "bf16")
    assert np.isfinite(out32).all()
    err = float(np.abs(out32 - ref).max())
    print(f"  max|err|={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("n,H", [(256, 12), (100, 8)])
def test_prefill_many_ragged_prompts(n, H):
    """More prompts than the workgroup ranks (prompts then run in index order,
    found by a prefix scan in chunks of 64): ragged lengths with empty,
    one-token and tile-multiple prompts, and a head count that leaves some XCD
    slices with fewer heads, against the oracle on every output."""
    rng = np.random.default_rng(90 + n)
    lens = [int(x) for x in rng.integers(0, 700, size=n)]
    lens[3], lens[10], lens[11], lens[77] = 0, 1, 128, 256
    print(f"prefill {n} prompts x {H} heads, total {sum(lens)}", flush=True)
    p = W.make_prefill(91, "bf16", H, 128, lens)
    out32 = down(_prefill(p))
    ref = oracle.attention.causal_prefill(p.q, p.k, p.v, p.prompt_lens, 1 / math.sqrt(128), "bf16")
    assert np.isfinite(out32).all()
    err = float(np.abs(out32 - ref).max())
    print(f"  max|err|={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_prefill_last_row_matches_decode():
    print("prefill <-> decode consistency", flush=True)
    dt, H, D, L = "bf16", 4, 128, 777
    p = W.make_prefill(72, dt, H, D, [L])
    out_p = down(_prefill(p))
    nb = -(-L // 16)
    kc = np.zeros((nb + 1, H, 16, D), np.uint16); vc = np.zeros_like(kc)
    table = np.random.default_rng(0).permutation(nb + 1).astype(np.int32)
    for t_ in range(L):
        kc[table[t_ // 16], :, t_ % 16] = p.k[t_]
        vc[table[t_ // 16], :, t_ % 16] = p.v[t_]
    d = W.DecodeInputs(name="consistency", dtype=dt, num_heads=H, head_dim=D, block_size=16, num_blocks=nb + 1,
                       scale=1 / math.sqrt(D), context_lens=np.array([L], np.int32), block_tables=table[None, :],
                       k_cache=kc, v_cache=vc, q=p.q[L - 1 : L].copy(), pad_block=int(table[nb]))
    out_d = down(run_decode(ops, upload_decode(d), d, "f32"))
    assert np.abs(out_p[L - 1] - out_d[0]).max() <= TOL[dt]


def test_mixed_step_config5():
    """Config 5 at full size: write (8 prompts + 192 decode tokens) -> prefill ->
    decode, then the same step with the prefill overlapped with write + decode
    on a second stream.  Every decode sequence and every prefill row and head is
    compared with the oracle."""
    print("mixed step config 5", flush=True)
    mx = W.mixed_config()
    d, p = mx.decode, mx.prefill
    B = 16
    # host bookkeeping: the prompts' slots, then the decode tokens' slots
    seq_p = np.repeat(np.arange(len(p.prompt_lens)), p.prompt_lens)
    pos_p = np.concatenate([np.arange(L) for L in p.prompt_lens])
    sm = np.concatenate([slot_mapping(p.block_tables, seq_p, pos_p, B),
                         slot_mapping(d.block_tables, np.arange(d.num_seqs), d.context_lens - 1, B)])
    sm_ref = np.concatenate([oracle.bookkeeping.slot_mapping(p.block_tables, seq_p, pos_p, B),
                             oracle.bookkeeping.slot_mapping(d.block_tables, range(d.num_seqs), d.context_lens - 1, B)])
    assert np.array_equal(sm, sm_ref)
    k_all = np.concatenate([p.k, d.k_new]); v_all = np.concatenate([p.v, d.v_new])
    mpl = int(p.prompt_lens.max())

    t = upload_decode(d)
    ops.kv_cache_write(up(k_all, d.dtype), up(v_all, d.dtype), up(sm), t["k_cache"], t["v_cache"])
    pout = nan_out(p.q.shape)
    ops.paged_attn_prefill(up(p.q, p.dtype), up(p.k, p.dtype), up(p.v, p.dtype), up(p.block_tables),
                           up(p.prompt_lens), pout, max_prompt_len=mpl)
    dout = run_decode(ops, t, d, "f32", partition_size=ops.PARTITION_AUTO)
    pout16 = nan_out(p.q.shape, p.dtype)
    ops.paged_attn_prefill(up(p.q, p.dtype), up(p.k, p.dtype), up(p.v, p.dtype), up(p.block_tables),
                           up(p.prompt_lens), pout16, max_prompt_len=mpl)
    torch.cuda.synchronize()

    # The same step with the prefill on a second stream, concurrent with the
    # write and the decode (they share no buffer): bit-identical results.
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    pout2 = nan_out(p.q.shape)
    side.wait_stream(main)
    with torch.cuda.stream(side):
        ops.paged_attn_prefill(up(p.q, p.dtype), up(p.k, p.dtype), up(p.v, p.dtype), up(p.block_tables),
                               up(p.prompt_lens), pout2, max_prompt_len=mpl)
    ops.kv_cache_write(up(k_all, d.dtype), up(v_all, d.dtype), up(sm), t["k_cache"], t["v_cache"])
    dout2 = run_decode(ops, t, d, "f32", partition_size=ops.PARTITION_AUTO)
    main.wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(pout, pout2) and torch.equal(dout, dout2)

    ek, ev = oracle.attention.cache_write(d.k_cache, d.v_cache, k_all, v_all, sm, B)
    assert np.array_equal(bits(down(t["k_cache"])), bits(ek))
    assert np.array_equal(bits(down(t["v_cache"])), bits(ev))
    del t
    record("config5", "kv_cache_write (8 prompts + 192 decode tokens)", max_abs_err=0.0, bit_exact_whole_pool=True,
           tokens=int(len(sm)), oracle_seconds=None)

    ref, t_dec = timed(oracle.attention.paged_decode, d.q, ek, ev, d.block_tables, d.context_lens, d.scale, d.dtype)
    got = down(dout)
    assert np.isfinite(got).all()
    derr = float(np.abs(got - ref).max())
    print(f"  decode max|err|={derr:.3e} (oracle {t_dec:.1f} s)", flush=True)
    assert derr <= TOL[d.dtype]
    record("config5", "paged_attn_decode (automatic partition)", max_abs_err=derr, tol=TOL[d.dtype],
           sequences=d.num_seqs, heads=d.num_heads, outputs_compared=int(dout.numel()),
           oracle_seconds=round(t_dec, 2))
    pref, t_pre = timed(oracle.attention.causal_prefill, p.q, p.k, p.v, p.prompt_lens, 1 / math.sqrt(p.head_dim),
                        p.dtype)
    pgot = down(pout)
    assert np.isfinite(pgot).all()
    perr = float(np.abs(pgot - pref).max())
    print(f"  prefill max|err|={perr:.3e} (oracle {t_pre:.1f} s)", flush=True)
    assert perr <= TOL[p.dtype]
    assert np.array_equal(bits(down(pout16)), bits(rne_to(pgot, p.dtype)))
    # raw error of the bf16 output against the oracle, and its bound 5e-3 + half an ulp of the oracle value
    p16 = oracle.attention.to_f64(down(pout16), p.dtype)
    half_ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(pref), np.abs(pgot)))[1] - 9)
    raw = np.abs(p16 - pref)
    assert (raw <= 5e-3 + half_ulp).all()
    record("config5", "paged_attn_prefill (8 prompts, 32 heads)", max_abs_err=perr, tol=TOL[p.dtype],
           prompts=int(len(p.prompt_lens)), tokens=int(p.prompt_lens.sum()), heads=p.num_heads,
           outputs_compared=int(pout.numel()), bit_exact_16bit_output_is_rne_of_f32=True,
           bf16_output_max_abs_err=float(raw.max()), oracle_seconds=round(t_pre, 2))


def _scatter_prompts(p, nb_extra=7, seed=0):
    """Write packed prompts into shuffled blocks through the host manager; returns tables and pools."""
    from paged_kv_cache_137_amd.blocks import BlockManager

    B = 16
    need = sum(-(-int(L) // B) for L in p.prompt_lens)
    nb = need + nb_extra
    m = BlockManager(nb, B, free_order=np.random.default_rng(seed).permutation(nb))
    slots = np.concatenate([m.add_sequence(i, int(L)) for i, L in enumerate(p.prompt_lens)])
    kc = W.normal((61, 1), (nb, p.num_heads, B, p.head_dim), p.dtype)
    vc = W.normal((61, 2), (nb, p.num_heads, B, p.head_dim), p.dtype)
    tk, tv = up(kc, p.dtype), up(vc, p.dtype)
    ops.kv_cache_write(up(p.k, p.dtype), up(p.v, p.dtype), up(slots), tk, tv)
    tables = m.block_tables(range(len(p.prompt_lens)), pad=0)
    return m, tables, tk, tv


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("f16", 64)])
def test_prefill_through_table_equals_contiguous(dt, D):
    print(f"paged prefill, no prefix, {dt} D={D}", flush=True)
    p = W.make_prefill(81, dt, 4, D, [1, 70, 200, 0, 129])
    _, tables, tk, tv = _scatter_prompts(p)
    a = _prefill(p)
    b = nan_out(a.shape, a.dtype)
    ops.paged_attn_prefill_cached(up(p.q, dt), tk, tv, up(tables), None, up(p.prompt_lens), b,
                                  max_prompt_len=int(p.prompt_lens.max()), max_prefix_len=0)
    assert torch.equal(a, b)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_prefill_over_shared_cached_prefix(dt):
    """Requests share a cached prefix (system prompt) through the same physical
    blocks; the partly filled last prefix block is copied on each request's
    first write; only the requests' own tokens run the prompt phase."""
    print(f"cached-prefix prefill {dt}", flush=True)
    from paged_kv_cache_137_amd.blocks import BlockManager

    H, D, B, nb = 8, 128, 16, 400
    rng = np.random.default_rng(5)
    m = BlockManager(nb, B, free_order=rng.permutation(nb))
    kc = W.normal((62, 1), (nb, H, B, D), dt)
    vc = W.normal((62, 2), (nb, H, B, D), dt)
    tk, tv = up(kc, dt), up(vc, dt)
    host_k, host_v = kc, vc
    # two cached prefixes: 300 tokens (ends inside a block) and 64 (whole blocks)
    prefixes = {100: 300, 200: 64}
    for sid, C in prefixes.items():
        k = W.normal((63, sid, 1), (C, H, D), dt); v = W.normal((63, sid, 2), (C, H, D), dt)
        sl = m.add_sequence(sid, C)
        ops.kv_cache_write(up(k, dt), up(v, dt), up(sl), tk, tv)
        host_k, host_v = oracle.attention.cache_write(host_k, host_v, k, v, sl, B)
    # requests: (prefix owner or None, new tokens)
    reqs = [(100, 1), (100, 129), (200, 77), (None, 40), (100, 513), (200, 16)]
    seqs, plens, prefs, new_slots = [], [], [], []
    for r, (owner, L) in enumerate(reqs):
        if owner is None:
            new_slots.append(m.add_sequence(r, L)); prefs.append(0)
        else:
            m.fork(owner, r); prefs.append(prefixes[owner])
            new_slots.append(np.asarray([m.append_token(r) for _ in range(L)], np.int64))
        seqs.append(r); plens.append(L)
    pairs = m.take_copies()
    assert len(pairs) == 3  # the 300-token prefix's partial block, once per request on it
    pr_ = np.asarray(pairs, np.int64)
    ops.copy_blocks(tk, tv, up(pr_))
    host_k, host_v = oracle.attention.copy_blocks(host_k, host_v, pr_)
    T = sum(plens)
    kn = W.normal((64, 1), (T, H, D), dt); vn = W.normal((64, 2), (T, H, D), dt); qn = W.normal((64, 3), (T, H, D), dt)
    sl = np.concatenate(new_slots)
    ops.kv_cache_write(up(kn, dt), up(vn, dt), up(sl), tk, tv)
    host_k, host_v = oracle.attention.cache_write(host_k, host_v, kn, vn, sl, B)
    tables = m.block_tables(seqs, pad=0)
    out = nan_out((T, H, D), torch.float32)
    ops.paged_attn_prefill_cached(up(qn, dt), tk, tv, up(tables), up(np.asarray(prefs, np.int32)),
                                  up(np.asarray(plens, np.int32)), out, max_prompt_len=max(plens),
                                  max_prefix_len=max(prefs))
    ref = oracle.attention.prefix_prefill(qn, host_k, host_v, tables, prefs, plens, 1 / math.sqrt(D), dt)
    got = down(out)
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    print(f"  max|err|={err:.3e}", flush=True)
    assert err <= TOL[dt]
    outdt = nan_out((T, H, D), TORCH_DT[dt])
    ops.paged_attn_prefill_cached(up(qn, dt), tk, tv, up(tables), up(np.asarray(prefs, np.int32)),
                                  up(np.asarray(plens, np.int32)), outdt, max_prompt_len=max(plens),
                                  max_prefix_len=max(prefs))
    assert np.array_equal(bits(down(outdt)), bits(rne_to(got, dt)))


@pytest.mark.parametrize("bs", [8, 32])
def test_cached_prefix_prefill_block_sizes(bs):
    print(f"cached-prefix prefill, block size {bs}", flush=True)
    from paged_kv_cache_137_amd.blocks import BlockManager

    dt, H, D, nb = "bf16", 4, 128, 300
    m = BlockManager(nb, bs, free_order=np.random.default_rng(bs).permutation(nb))
    kc = W.normal((65, bs, 1), (nb, H, bs, D), dt)
    vc = W.normal((65, bs, 2), (nb, H, bs, D), dt)
    tk, tv = up(kc, dt), up(vc, dt)
    C = 3 * bs + 5
    k = W.normal((66, bs, 1), (C, H, D), dt); v = W.normal((66, bs, 2), (C, H, D), dt)
    sl = m.add_sequence(-1, C)
    ops.kv_cache_write(up(k, dt), up(v, dt), up(sl), tk, tv)
    hk, hv = oracle.attention.cache_write(kc, vc, k, v, sl, bs)
    plens = [7, 130]
    slots = []
    for r, L in enumerate(plens):
        m.fork(-1, r)
        slots.append(np.asarray([m.append_token(r) for _ in range(L)], np.int64))
    pairs = np.asarray(m.take_copies(), np.int64)
    ops.copy_blocks(tk, tv, up(pairs))
    hk, hv = oracle.attention.copy_blocks(hk, hv, pairs)
    T = sum(plens)
    kn = W.normal((67, bs, 1), (T, H, D), dt); vn = W.normal((67, bs, 2), (T, H, D), dt)
    qn = W.normal((67, bs, 3), (T, H, D), dt)
    sl = np.concatenate(slots)
    ops.kv_cache_write(up(kn, dt), up(vn, dt), up(sl), tk, tv)
    hk, hv = oracle.attention.cache_write(hk, hv, kn, vn, sl, bs)
    tables = m.block_tables(range(len(plens)), pad=0)
    out = nan_out((T, H, D), torch.float32)
    ops.paged_attn_prefill_cached(up(qn, dt), tk, tv, up(tables), up(np.full(len(plens), C, np.int32)),
                                  up(np.asarray(plens, np.int32)), out, max_prompt_len=max(plens), max_prefix_len=C)
    ref = oracle.attention.prefix_prefill(qn, hk, hv, tables, [C] * len(plens), plens, 1 / math.sqrt(D), dt,
                                          block_size=bs)
    assert np.abs(down(out) - ref).max() <= TOL[dt]


def test_cached_prefix_prefill_long_prefix():
    """Two requests of 200 and 77 new tokens over one 16,384-token cached prefix
    (1,024 shared blocks, then each request's own), read through shuffled
    tables, bf16, 4 heads x 128: every output against the oracle."""
    print("cached-prefix prefill, 16,384-token prefix", flush=True)
    dt, H, D, bs, C = "bf16", 4, 128, 16, 16384
    plens = [200, 77]
    need = [-(-(C + L) // bs) for L in plens]
    npre = C // bs
    nb = npre + sum(n - npre for n in need) + 8
    perm = np.random.default_rng(9).permutation(nb).astype(np.int32)
    tables = np.zeros((len(plens), max(need)), np.int32)
    o = npre
    for r, n in enumerate(need):
        tables[r, :npre] = perm[:npre]
        tables[r, npre:n] = perm[o:o + n - npre]
        o += n - npre
    kc = W.normal((69, 1), (nb, H, bs, D), dt)
    vc = W.normal((69, 2), (nb, H, bs, D), dt)
    T = sum(plens)
    qn = W.normal((69, 3), (T, H, D), dt)
    out = nan_out((T, H, D), torch.float32)
    ops.paged_attn_prefill_cached(up(qn, dt), up(kc, dt), up(vc, dt), up(tables), up(np.full(len(plens), C, np.int32)),
                                  up(np.asarray(plens, np.int32)), out, max_prompt_len=max(plens), max_prefix_len=C)
    ref = oracle.attention.prefix_prefill(qn, kc, vc, tables, [C] * len(plens), plens, 1 / math.sqrt(D), dt,
                                          block_size=bs)
    got = down(out)
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    print(f"  max|err|={err:.3e}", flush=True)
    assert err <= TOL[dt]


@pytest.mark.parametrize("bs,D", [(16, 128), (8, 64)])
def test_cached_prefix_prefill_bad_id_poisons_later_queries(bs, D):
    """A table entry outside the pool is never read: every query that would see
    that block gets NaN, the earlier queries are exact."""
    print(f"cached-prefix prefill bad id, block size {bs}, D={D}", flush=True)
    dt, H, nb, C, L = "bf16", 4, 40, 40, 100
    nblk = -(-(C + L) // bs)
    rng = np.random.default_rng(7)
    table = rng.permutation(nb)[:nblk].astype(np.int32)[None, :]
    kc = W.normal((68, 1), (nb, H, bs, D), dt)
    vc = W.normal((68, 2), (nb, H, bs, D), dt)
    qn = W.normal((68, 3), (L, H, D), dt)
    jb = 96 // bs  # the block holding key position 96
    bad = table.copy()
    bad[0, jb] = nb + 5
    out = nan_out((L, H, D), torch.float32, fill=7.0)  # a finite fill: the NaN must come from the kernel
    ops.paged_attn_prefill_cached(up(qn, dt), up(kc, dt), up(vc, dt), up(bad), up(np.asarray([C], np.int32)),
                                  up(np.asarray([L], np.int32)), out, max_prompt_len=L, max_prefix_len=C)
    got = down(out)
    first_bad = jb * bs - C  # first query (new-token index) whose keys reach the bad block
    assert np.isnan(got[first_bad:]).all()
    ref = oracle.attention.prefix_prefill(qn, kc, vc, table, [C], [L], 1 / math.sqrt(D), dt, block_size=bs)
    assert np.isfinite(got[:first_bad]).all()
    assert np.abs(got[:first_bad] - ref[:first_bad]).max() <= TOL[dt]
