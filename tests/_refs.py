"""Float64 oracle results for the full-size configurations, computed once per
test session and shared by the tests that check them (the plain and the
shared-prefix decode of config 4 compare against the same reference)."""

from __future__ import annotations

import oracle
from _dev import timed

_DECODE: dict = {}


def decode_ref(key, d, kc=None, vc=None):
    """(oracle.attention.paged_decode over every sequence of d, seconds it took).

    `key` names the inputs (for instance the config number): the first call for
    a key computes, later calls return the stored result.  kc/vc replace d's
    pools (for instance after a cache write)."""
    if key not in _DECODE:
        _DECODE[key] = timed(oracle.attention.paged_decode, d.q, d.k_cache if kc is None else kc,
                             d.v_cache if vc is None else vc, d.block_tables, d.context_lens, d.scale, d.dtype,
                             block_size=d.block_size)
    return _DECODE[key]
