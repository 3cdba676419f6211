"""Float64 CPU oracle for exact attention and Flash-Decoding.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, constants or helpers with the HIP
library under ``exact_io_aware_02_amd/``; the two meet only through seeded
inputs made by ``synth``.

Sources (three web pages on one subject; cited by title and section):

* "Infra: Flash Attention" (pufanyi.com blog), sections "Attention and scope",
  "Online softmax and state merging" (stable normalisation; merging block
  states; accumulating the attention weighted sum, with the 49/15 worked
  example), "Tiled computation and forward" (Algorithm 1 and the boundary
  conditions), "Backward and recomputation" (definition of L).
* The airsota interview card on efficient attention / Flash-Decoding,
  section 3 "Mathematical principles & derivation" (Flash-Decoding steps 1-3:
  sequence partitioning, per-chunk partials, log-sum-exp reduction).
* "CMU 10-423 Lecture 18: FlashAttention & efficient decoding" notes,
  sections 2.1-2.3 (online softmax, (m, l, o) merging), 3.2-3.4 (tiled forward,
  FA-2 loop order), 4.1 and 4.3 (IO counts, causal tile skipping), 5.3 (the
  FlashAttention backward by recomputation), 7.3 (KV cache in blocks behind
  a block table) and Exercises 1-4.

Modules:

* ``attention``  -- the plain definition: O = softmax(Q K^T * scale) V and
  L = log-sum-exp per row, causal or not, plus the single-query decode form,
  and the P-weighted spread of V around O (a bound on the effect of rounding
  P before the product with V).
* ``online``     -- scalar online softmax, the (m, l, u) block state and its
  merge, and the Flash-Decoding combine of (O^(k), m^(k), l^(k)) partials.
* ``tiled``      -- Algorithm 1 of "Infra: Flash Attention" taken step by step
  with tile counters, and the closed-form IO counts of the lecture notes.
* ``backward``   -- gradients dQ, dK, dV of exact attention: the plain
  definition through P, and the tiled recomputation from O and L
  ("Infra: Flash Attention", "Backward and recomputation").
* ``paged``      -- decode against a KV cache kept in fixed-size blocks and
  read through a block table (lecture notes, section 7.3), both as the plain
  definition on the gathered cache and block by block with (m, l, u) merges.

Parity status: every function here is pinned by a CPU test under ``tests/``
(values printed on the pages, closed forms, a library routine, or brute force).
None is "parity unpinned".
"""

from .attention import attention_ref, attention_rows, attention_dev_rows, decode_ref
from .online import (
    online_softmax,
    block_state,
    merge,
    finalize,
    combine_partials,
    per_block_softmax,
)
from .tiled import tiled_ref, io_standard, io_fa2, io_fa1_main, causal_tile_count
from .paged import blocks_of, gather_paged, decode_paged_ref, decode_paged_blockwise
from .backward import attention_backward, attention_backward_ref, attention_backward_tiled

__all__ = [
    "attention_ref",
    "attention_rows",
    "attention_dev_rows",
    "decode_ref",
    "online_softmax",
    "block_state",
    "merge",
    "finalize",
    "combine_partials",
    "per_block_softmax",
    "tiled_ref",
    "io_standard",
    "io_fa2",
    "io_fa1_main",
    "causal_tile_count",
    "blocks_of",
    "gather_paged",
    "decode_paged_ref",
    "decode_paged_blockwise",
    "attention_backward",
    "attention_backward_ref",
    "attention_backward_tiled",
]
