"""kv_cache_write on the GPU against the oracle's byte copy: bit-exact, the whole pool."""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_137_amd import ops
from paged_kv_cache_137_amd import workloads as W
from _dev import bits, down, up

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt,H,D", [("bf16", 32, 128), ("f16", 40, 128), ("f32", 4, 64), ("bf16", 8, 64), ("f32", 2, 128)])
def test_write_matches_oracle_bit_exact(dt, H, D):
    print(f"write parity {dt} H={H} D={D}", flush=True)
    rng = np.random.default_rng(1)
    nb, T = 300, 1000
    kc = W.normal((5, 1), (nb, H, 16, D), dt)
    vc = W.normal((5, 2), (nb, H, 16, D), dt)
    kc[rng.integers(0, nb, 50), :, rng.integers(0, 16, 50), :] = W.nan_value(dt)  # canaries
    k = W.normal((5, 3), (T, H, D), dt)
    v = W.normal((5, 4), (T, H, D), dt)
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    slots[rng.integers(0, T, 37)] = -1  # padding tokens
    tk, tv = up(kc, dt), up(vc, dt)
    ops.kv_cache_write(up(k, dt), up(v, dt), up(slots), tk, tv)
    ek, ev = oracle.attention.cache_write(kc, vc, k, v, slots, 16)
    assert np.array_equal(bits(down(tk)), bits(ek))
    assert np.array_equal(bits(down(tv)), bits(ev))


def test_write_skips_out_of_pool_slots_and_empty_batch():
    print("write guards", flush=True)
    dt, H, D, nb = "bf16", 4, 128, 8
    kc = W.normal((6, 1), (nb, H, 16, D), dt)
    k = W.normal((6, 2), (3, H, D), dt)
    slots = np.array([nb * 16, nb * 16 + 5, 2**40], dtype=np.int64)  # all outside the pool
    tk, tv = up(kc, dt), up(kc, dt)
    ops.kv_cache_write(up(k, dt), up(k, dt), up(slots), tk, tv)
    ops.kv_cache_write(up(k[:0], dt), up(k[:0], dt), up(slots[:0]), tk, tv)
    torch.cuda.synchronize()
    assert np.array_equal(bits(down(tk)), bits(kc)) and np.array_equal(bits(down(tv)), bits(kc))


def test_write_then_gather_returns_the_new_tokens():
    print("write then gather", flush=True)
    d = W.make_decode(21, "f16", 40, 128, [1, 15, 16, 17, 33, 700], with_new_tokens=True)
    from paged_kv_cache_137_amd.blocks import slot_mapping

    sm = slot_mapping(d.block_tables, range(d.num_seqs), d.context_lens - 1)
    assert np.array_equal(sm, oracle.bookkeeping.slot_mapping(d.block_tables, range(d.num_seqs), d.context_lens - 1, 16))
    tk, tv = up(d.k_cache, "f16"), up(d.v_cache, "f16")
    ops.kv_cache_write(up(d.k_new, "f16"), up(d.v_new, "f16"), up(sm), tk, tv)
    gk, gv = down(tk), down(tv)
    for s in range(d.num_seqs):
        n = int(d.context_lens[s])
        assert np.array_equal(bits(oracle.attention.gather(gk, d.block_tables[s], n, 16)[:, n - 1]), bits(d.k_new[s]))
        assert np.array_equal(bits(oracle.attention.gather(gv, d.block_tables[s], n, 16)[:, n - 1]), bits(d.v_new[s]))
