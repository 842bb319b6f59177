"""CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check of the package entry
file and the bench's CPU-baseline leg may import or run anything in this
package; the library and its Python binding never do, and there is no CPU
fallback anywhere in the product path.  It shares no code with the HIP path:
inputs come from the seeded generators in ``workloads`` and from nothing else.

Contents and what pins each part (tests/test_oracle.py):

* ``paged_attention`` - KV write, gather through block tables, bottom-right
  causal softmax attention, prefill, decode, split-K partials and their merge.
  Pinned by a hand-worked golden store fixture, pure-Python brute force on
  contiguous unpaged K/V, torch's CPU scaled_dot_product_attention in float64,
  closed forms (one key, equal keys, one-hot probes), invariance under block
  relabelling / prefix copies / stale poisoning, decode == last prefill row,
  split merge == unsplit, float32 vs float64 agreement, and planted mistakes
  that each of those must catch.
* ``block_manager`` - the pages' block allocation (a fixed pool of ids with
  reference counts, a first-in first-out queue of free ids, prefix sharing) and
  the step planner.  Pinned by hand-worked allocation
  fixtures, reference-count and exhaustion invariants, and slot round trips.
  ``PrefixCache`` models the prefix-cached manager keyed by whole token prefixes;
  pinned by the hand-worked scenarios of tests/test_block_manager.py and the
  reference-count / free-deque / registration invariants checked there.
* ``step`` - a whole step (writes, then prefill and decode) on plain arrays.
* ``rotary`` - rotary position embedding (RoFormer's pair rotation, half-split
  pairing) and a round-to-nearest-even bf16 rounding from its definition; pinned by
  tests/test_rotary_oracle.py (identity at position 0, a hand-worked pair rotation,
  pair norms, inverse and composition, relative-position scores, RNE ties).

Everything is float64 unless a caller asks for float32; nothing is tuned.
"""
from .block_manager import IdPool, PrefixCache, cumulative_lengths, plan_step, slot_of
from .paged_attention import (as_float, bf16_bits_to_float, causal_attention, combine_partials,
                              decode_split_partials, gather_tokens, kv_head_of, paged_decode,
                              paged_prefill, store_kvcache)
from .step import build_caches, run_step, stale_value
