"""Plain, slow CPU oracle for the paged KV-cache attention path.

TEST INFRASTRUCTURE ONLY.  Only the tests under tests/, the smoke check in
__graft_entry__.py and the CPU-baseline leg of bench.py may import or run this
package.  The product path (the HIP library and its Python binding) never calls
it and never falls back to it.  It shares no code with that path.  It is written
directly from the pages' definitions, in float64, with no blocking or fusion.

Sources (the pages this reproduces), cited by title and section:
  "PagedAttention and vLLM, annotated"
  "vLLM & PagedAttention: Efficient Memory Management for LLM Serving"
  (shortened to "vLLM & PagedAttention" after the first mention in a file)

Modules:
  bookkeeping  block counts, slot numbering, per-token KV bytes (integer, exact)
  attention    cache write (byte copy), paged decode, causal prefill (float64)

Parity pins: every function here is pinned in tests/test_oracle_pins.py
against printed worked examples, closed forms, invariants and an independent
library routine.  No function is "parity unpinned".
"""

from . import attention, bookkeeping  # noqa: F401
