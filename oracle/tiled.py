"""Algorithm 1 of "Infra: Flash Attention" taken step by step, in float64,
with tile and traffic counters; and the closed-form HBM access counts of the
"CMU 10-423 Lecture 18" notes.

TEST INFRASTRUCTURE ONLY (see the package docstring).  This module exists to
pin the algebra of tiling against the plain definition in ``attention``; it
is never the parity reference for the GPU path.

Algorithm 1 ("Infra: Flash Attention", section "Tiled computation and
forward"), FlashAttention-2 order (query tile outer, KV tile inner):

    for each query tile Q_i:
        m = -inf, l = 0, U = 0
        for each KV tile (K_j, V_j):
            S = Q_i K_j^T * scale
            mask S; a row with every score of this tile masked skips the update
            m' = max(m, rowmax S); alpha = exp(m - m'); W = exp(S - m')
            l = alpha l + rowsum W; U = alpha U + W V_j; m = m'
        O_i = U / l;  L_i = m + log l

Causal tiles that lie wholly in the future of every query of the tile are not
visited at all; tiles crossing the diagonal are masked on chip (same page,
figure on causal tiles; the lecture notes, section 4.3).

Traffic model ("CMU 10-423 Lecture 18", section 4.1 and Exercise 3): Q_i is
read once per query tile, K_j and V_j once per visited (i, j) pair, O_i and
L_i written once.  For a full non-causal pass this is
N d + 2 N d (N / B_r) + N d + N elements.
"""

import numpy as np


def tiled_ref(Q, K, V, Br, Bc, scale, causal=False, count=False):
    """One head: Q, K [N, d], V [N, dv].  Returns (O, L) or, with count=True,
    (O, L, counters) where counters = {"tiles", "reads", "writes"} in
    elements under the model above."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    N, d = Q.shape
    Nk = K.shape[0]
    dv = V.shape[1]
    O = np.zeros((N, dv))
    L = np.full((N,), -np.inf)
    tiles = reads = writes = 0
    for q0 in range(0, N, Br):
        q1 = min(N, q0 + Br)
        Qi = Q[q0:q1]
        reads += Qi.size
        rows = q1 - q0
        qpos = np.arange(q0, q1)
        m = np.full((rows,), -np.inf)
        l = np.zeros((rows,))
        U = np.zeros((rows, dv))
        for k0 in range(0, Nk, Bc):
            if causal and k0 > q1 - 1:
                break  # this tile and every later one lies in the future
            k1 = min(Nk, k0 + Bc)
            Kj, Vj = K[k0:k1], V[k0:k1]
            tiles += 1
            reads += Kj.size + Vj.size
            S = (Qi @ Kj.T) * scale
            if causal:
                kpos = np.arange(k0, k1)
                S = np.where(kpos[None, :] <= qpos[:, None], S, -np.inf)
            live = np.isfinite(S).any(axis=1)  # rows with a valid key here
            if not live.any():
                continue
            Sl = S[live]
            m_new = np.maximum(m[live], Sl.max(axis=1))
            alpha = np.where(np.isfinite(m[live]), np.exp(m[live] - m_new), 0.0)
            W = np.exp(Sl - m_new[:, None])
            l[live] = alpha * l[live] + W.sum(axis=1)
            U[live] = alpha[:, None] * U[live] + W @ Vj
            m[live] = m_new
        done = l > 0
        O[q0:q1][done] = U[done] / l[done][:, None]
        L[q0:q1][done] = m[done] + np.log(l[done])
        writes += rows * dv + rows
    if count:
        return O, L, {"tiles": tiles, "reads": reads, "writes": writes}
    return O, L


def io_standard(N, d):
    """Forward HBM element accesses of three-kernel attention: S written and
    read, P written and read, plus Q, K, V read and O written: 4N^2 + 4Nd
    ("CMU 10-423 Lecture 18", section 4.1)."""
    return 4 * N * N + 4 * N * d


def io_fa2(N, d, Br):
    """FlashAttention-2 order: Q read once, K and V read once per query tile,
    O written once, plus the N log-sum-exp values (section 4.1, Exercise 3)."""
    Tr = -(-N // Br)
    return N * d + 2 * N * d * Tr + N * d + N


def io_fa1_main(N, d, M):
    """Leading term 12 N^2 d^2 / M of the KV-outer (FlashAttention-1) order
    with B_c = M / (4d): each of the N/B_c KV tiles reads Q and O and writes O
    (3Nd elements) (section 4.1)."""
    return 12 * N * N * d * d / M


def causal_tile_count(T):
    """Tiles visited by causal attention with T query tiles and T KV tiles of
    equal size: query tile i needs KV tiles 1..i, so T(T+1)/2 in total
    ("CMU 10-423 Lecture 18", Exercise 4)."""
    return T * (T + 1) // 2
