"""A KV cache kept in fixed-size blocks and read through a block table, in
float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"CMU 10-423 Lecture 18" notes, section 7.3: the KV cache is cut into blocks
that each hold a fixed number of tokens; a sequence's blocks need not be
contiguous, a block table maps its logical block i to a physical block, and
attention is computed block by block, the blocks' partial results merged with
the (m, l, o) state of section 2.3.  Only a sequence's last block may be
partly filled.

Layout taken here (the page fixes none): one pool per K and V, shaped
[num_blocks, H, block_size, d]; physical block p holds block_size consecutive
tokens of every head.  table[b, i] is the physical block of sequence b's
logical block i, for i < ceil(L_b / block_size); later entries are never read.

* ``gather_paged``           -- the contiguous cache [H, L_b, d] of one sequence.
* ``decode_paged_ref``       -- the plain definition: single-query attention
  (``decode_ref``) over the gathered cache, for every (b, h).
* ``decode_paged_blockwise`` -- the page's procedure for one (b, h): one
  (m, l, u) state per block, read straight from the pool, merged left to right.
"""

import numpy as np

from .attention import decode_ref
from .online import block_state, finalize, merge


def blocks_of(length, block_size):
    """Logical blocks a sequence of `length` tokens occupies."""
    return -(-int(length) // int(block_size))


def gather_paged(pool, table_row, length, block_size):
    """Contiguous cache [H, length, d] of one sequence from a pool
    [num_blocks, H, block_size, d] and its row of the block table."""
    pool = np.asarray(pool)
    H, d = pool.shape[1], pool.shape[3]
    nb = blocks_of(length, block_size)
    if nb == 0:
        return np.zeros((H, 0, d), dtype=np.float64)
    parts = [np.asarray(pool[int(table_row[i])], dtype=np.float64) for i in range(nb)]
    return np.concatenate(parts, axis=1)[:, : int(length)]


def decode_paged_ref(q, Kpool, Vpool, table, lengths, block_size, scale, pairs=None):
    """Decode of q [B, H, d] against paged caches.  Returns float64
    (o [B, H, d], lse [B, H]); an empty sequence gives o = 0, lse = -inf.
    `pairs` optionally restricts the work to a list of (b, h); other entries
    are left at zero / nan."""
    q = np.asarray(q, dtype=np.float64)
    B, H, d = q.shape
    o = np.zeros((B, H, d), dtype=np.float64)
    lse = np.full((B, H), np.nan)
    todo = pairs if pairs is not None else [(b, h) for b in range(B) for h in range(H)]
    gathered = {}
    for b, h in todo:
        if b not in gathered:
            gathered[b] = (
                gather_paged(Kpool, table[b], lengths[b], block_size),
                gather_paged(Vpool, table[b], lengths[b], block_size),
            )
        Kb, Vb = gathered[b]
        o[b, h], lse[b, h] = decode_ref(q[b, h], Kb[h], Vb[h], scale)
    return o, lse


def decode_paged_blockwise(q_bh, Kpool, Vpool, table_row, length, block_size, h, scale):
    """One (b, h) computed block by block: the scores of each physical block's
    valid tokens form an (m, l, u) state, the states are merged in logical
    order, and the merged state is finalised.  Returns (o [d], lse)."""
    q_bh = np.asarray(q_bh, dtype=np.float64)
    d = q_bh.shape[0]
    state = (-np.inf, 0.0, np.zeros(d))
    for i in range(blocks_of(length, block_size)):
        p = int(table_row[i])
        n = min(int(block_size), int(length) - i * int(block_size))
        k = np.asarray(Kpool[p, h, :n], dtype=np.float64)
        v = np.asarray(Vpool[p, h, :n], dtype=np.float64)
        state = merge(state, block_state((k @ q_bh) * scale, v))
    return finalize(state)
