"""Pins for the paged-KV decode oracle ("CMU 10-423 Lecture 18" notes, section
7.3): the block table reproduces the contiguous cache exactly, computing
block by block with (m, l, o) merges agrees with the contiguous computation
to float64 rounding, and neither depends on where the blocks sit."""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "paged_blocks_section73.json")


def _scatter(contig, block_size, phys_ids, num_blocks, rng):
    """Pool [num_blocks, H, bs, d] holding contig [H, L, d] at the given
    physical blocks; every other slot is filled with noise."""
    H, L, d = contig.shape
    pool = rng.standard_normal((num_blocks, H, block_size, d)) * 100.0
    for i, p in enumerate(phys_ids):
        n = min(block_size, L - i * block_size)
        pool[p, :, :n] = contig[:, i * block_size: i * block_size + n]
    return pool


def test_worked_example_section73():
    g = json.load(open(GOLDEN))
    bs, nblk = g["block_size"], g["num_blocks"]
    tables = {"A": [0, 2, 3], "B": g["request_B_table"], "C": [6, 7]}
    lengths = {"A": 11, "B": 10, "C": 5}
    assert tables["B"] == [1, 4, 5]
    rng = np.random.default_rng(73)
    H, d = 2, 8
    for name in tables:
        assert len(tables[name]) == oracle.blocks_of(lengths[name], bs)
    used = sorted(p for t in tables.values() for p in t)
    assert len(used) == len(set(used)) and max(used) < nblk
    K = {n: rng.standard_normal((H, lengths[n], d)) for n in tables}
    V = {n: rng.standard_normal((H, lengths[n], d)) for n in tables}
    Kpool = rng.standard_normal((nblk, H, bs, d))
    Vpool = rng.standard_normal((nblk, H, bs, d))
    for n, t in tables.items():
        for i, p in enumerate(t):
            c = min(bs, lengths[n] - i * bs)
            Kpool[p, :, :c] = K[n][:, i * bs: i * bs + c]
            Vpool[p, :, :c] = V[n][:, i * bs: i * bs + c]
    for n, t in tables.items():
        # the K gathered through the table is exactly the stored K
        assert np.array_equal(oracle.gather_paged(Kpool, t, lengths[n], bs), K[n])
        q = rng.standard_normal((d,))
        for h in range(H):
            o_c, l_c = oracle.decode_ref(q, K[n][h], V[n][h], 0.5)
            o_b, l_b = oracle.decode_paged_blockwise(q, Kpool, Vpool, t, lengths[n], bs, h, 0.5)
            assert np.abs(o_b - o_c).max() <= 10 * g["printed_difference"] * max(1.0, np.abs(o_c).max())
            assert abs(l_b - l_c) <= 1e-14
    # waste sits only in each request's last block: at most bs - 1 slots
    for n in tables:
        assert len(tables[n]) * bs - lengths[n] <= bs - 1


@pytest.mark.parametrize("bs", [1, 4, 16, 64])
@pytest.mark.parametrize("L", [0, 1, 15, 16, 17, 200])
def test_gather_is_exact_and_blockwise_matches_plain(bs, L):
    rng = np.random.default_rng(1000 * bs + L)
    H, d = 3, 16
    contig = rng.standard_normal((H, L, d))
    vals = rng.standard_normal((H, L, d))
    nb = oracle.blocks_of(L, bs)
    num_blocks = nb + 5
    phys = rng.permutation(num_blocks)[:nb]
    Kpool = _scatter(contig, bs, phys, num_blocks, rng)
    Vpool = _scatter(vals, bs, phys, num_blocks, rng)
    assert np.array_equal(oracle.gather_paged(Kpool, phys, L, bs), contig)
    q = rng.standard_normal((1, H, d))
    o, lse = oracle.decode_paged_ref(q, Kpool, Vpool, phys[None], [L], bs, 0.25)
    for h in range(H):
        o_c, l_c = oracle.decode_ref(q[0, h], contig[h], vals[h], 0.25)
        assert np.array_equal(o[0, h], o_c) and (lse[0, h] == l_c)
        o_b, l_b = oracle.decode_paged_blockwise(q[0, h], Kpool, Vpool, phys, L, bs, h, 0.25)
        if L == 0:
            assert l_b == -np.inf and np.all(o_b == 0)
        else:
            assert np.abs(o_b - o_c).max() <= 1e-13 and abs(l_b - l_c) <= 1e-13


def test_physical_placement_does_not_matter():
    """Moving blocks to other physical slots (and updating the table) leaves
    the result bitwise unchanged: it depends on the gathered cache only."""
    rng = np.random.default_rng(5)
    B, H, d, bs = 3, 2, 8, 4
    lengths = [9, 0, 13]
    nbs = [oracle.blocks_of(L, bs) for L in lengths]
    num_blocks = sum(nbs) + 3
    Kpool = rng.standard_normal((num_blocks, H, bs, d))
    Vpool = rng.standard_normal((num_blocks, H, bs, d))
    perm = rng.permutation(num_blocks)
    table = np.full((B, max(nbs)), -1)
    k = 0
    for b, n in enumerate(nbs):
        table[b, :n] = perm[k:k + n]
        k += n
    q = rng.standard_normal((B, H, d))
    o1, l1 = oracle.decode_paged_ref(q, Kpool, Vpool, table, lengths, bs, 0.3)
    move = rng.permutation(num_blocks)          # block p goes to slot move[p]
    K2 = np.empty_like(Kpool); V2 = np.empty_like(Vpool)
    K2[move] = Kpool; V2[move] = Vpool
    table2 = np.where(table >= 0, move[np.maximum(table, 0)], -1)
    o2, l2 = oracle.decode_paged_ref(q, K2, V2, table2, lengths, bs, 0.3)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.all(o1[1] == 0) and np.all(l1[1] == -np.inf)


def test_slots_past_the_end_are_never_read():
    rng = np.random.default_rng(9)
    H, d, bs, L = 2, 8, 16, 21            # last block holds 5 tokens
    Kpool = rng.standard_normal((4, H, bs, d))
    Vpool = rng.standard_normal((4, H, bs, d))
    table = np.array([[3, 1]])
    q = rng.standard_normal((1, H, d))
    o1, l1 = oracle.decode_paged_ref(q, Kpool, Vpool, table, [L], bs, 0.5)
    Kpool[1, :, 5:] = np.nan
    Vpool[1, :, 5:] = np.nan
    Kpool[[0, 2]] = np.nan                 # blocks outside the table
    o2, l2 = oracle.decode_paged_ref(q, Kpool, Vpool, table, [L], bs, 0.5)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    for h in range(H):
        o_b, _ = oracle.decode_paged_blockwise(q[0, h], Kpool, Vpool, table[0], L, bs, h, 0.5)
        assert np.all(np.isfinite(o_b))
