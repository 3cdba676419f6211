"""Gradients of exact attention with respect to Q, K and V, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, per head, given the upstream gradient G = dLoss/dO
("Infra: Flash Attention", sections "Backward and recomputation" and the
tiled-gradient section after it; "CMU 10-423 Lecture 18" notes, section 5.3):

    S = Q K^T * scale, causal keys after the query masked to -inf
    P = row softmax of S                       (the forward's probabilities)
    dV = P^T G
    H  = dP = G V^T
    D_i = sum_j P_ij H_ij                      (the softmax Jacobian term)
    dS_ij = P_ij (H_ij - D_i)                  (row-wise softmax backward)
    dQ = scale * dS K
    dK = scale * dS^T Q

The blog writes the scale as 1/sqrt(d); a general scale enters the chain
rule the same way (S is linear in it).  The pages also rewrite D_i as
G_i . O_i (O = P V), which needs no pass over P; the plain definition above
forms D from P and H, and a pin checks that the two agree.

``attention_backward`` is that definition: whole rows of P are formed (a
block of query rows at a time only to bound memory; dK and dV add up the
blocks' contributions).  ``attention_backward_tiled`` follows the tiled
procedure the pages describe instead: the forward keeps only O and the
per-row log-sum-exp L; the backward walks KV tiles, recomputes each tile's
probabilities as P_ij = exp(S_ij - L_i), takes D from G and O, and adds each
tile's contributions to dQ, dK and dV.  It exists to pin the algebra of the
tiled form against the definition, as ``tiled_ref`` does for the forward.

A row with no valid key (unreachable for square causal attention) gets
P = 0, so it contributes nothing and its dQ row is 0.
"""

import numpy as np

from .attention import attention_rows

_ROW_BLOCK_ELEMS = 1 << 22  # at most 4M float64 scores per block of rows


def _masked_scores(q, k, scale, causal, q_pos):
    s = (q @ k.T) * scale
    if causal:
        key_pos = np.arange(k.shape[0])
        s = np.where(key_pos[None, :] <= q_pos[:, None], s, -np.inf)
    return s


def _softmax_rows(s):
    """Row softmax of masked scores; an all-masked row gives zeros."""
    m = s.max(axis=1)
    valid = np.isfinite(m)
    p = np.exp(s - np.where(valid, m, 0.0)[:, None])
    l = p.sum(axis=1)
    return p / np.where(valid, l, 1.0)[:, None]


def _row_D(p, h):
    """D_i = sum_j P_ij H_ij."""
    return (p * h).sum(axis=1)


def _score_grad(p, h, D):
    """dS_ij = P_ij (H_ij - D_i)."""
    return p * (h - D[:, None])


def attention_backward(q, k, v, do, scale, causal=False):
    """Gradients of one head: q [N, d], k [Nk, d], v [Nk, dv], do [N, dv]
    (the upstream gradient of O).  Causal keeps key j for query i iff j <= i.
    Returns float64 (dQ [N, d], dK [Nk, d], dV [Nk, dv], D [N])."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    N = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    D = np.zeros((N,), dtype=np.float64)
    rb = max(1, _ROW_BLOCK_ELEMS // max(1, k.shape[0]))
    for r0 in range(0, N, rb):
        r1 = min(N, r0 + rb)
        p = _softmax_rows(_masked_scores(q[r0:r1], k, float(scale), causal, np.arange(r0, r1)))
        h = do[r0:r1] @ v.T
        Db = _row_D(p, h)
        ds = _score_grad(p, h, Db)
        dq[r0:r1] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r0:r1])
        dv += p.T @ do[r0:r1]
        D[r0:r1] = Db
    return dq, dk, dv, D


def attention_backward_ref(Q, K, V, dO, scale, causal=False):
    """attention_backward over arrays shaped [..., N, d] (any leading
    batch/head dims).  Returns float64 (dQ, dK, dV)."""
    Q, K, V, dO = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, dO))
    lead = Q.shape[:-2]
    dq, dk, dv = np.empty_like(Q), np.empty_like(K), np.empty_like(V)
    for idx in np.ndindex(*lead):
        dq[idx], dk[idx], dv[idx], _ = attention_backward(Q[idx], K[idx], V[idx], dO[idx], scale, causal)
    return dq, dk, dv


def attention_backward_tiled(q, k, v, do, scale, block_rows, block_cols, causal=False, o=None, lse=None):
    """The tiled backward of the pages, taken step by step, for one head.

    The forward's O and L (natural-log log-sum-exp per row) are computed by
    the plain forward unless given.  D_i = G_i . O_i.  For each KV tile j and
    each query tile i that has a key not in its future: S = Q_i K_j^T scale
    (masked), P = exp(S - L_i), dV_j += P^T G_i, H = G_i V_j^T,
    dS = P (H - D_i), dQ_i += scale dS K_j, dK_j += scale dS^T Q_i.
    Returns float64 (dQ, dK, dV)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    N, Nk = q.shape[0], k.shape[0]
    if o is None or lse is None:
        o, lse = attention_rows(q, k, v, scale, causal=causal)
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    D = (do * o).sum(axis=1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for j0 in range(0, Nk, block_cols):
        j1 = min(Nk, j0 + block_cols)
        for i0 in range(0, N, block_rows):
            i1 = min(N, i0 + block_rows)
            if causal and j0 > i1 - 1:
                continue  # every key of this tile is after every query of it
            s = _masked_scores(q[i0:i1], k[j0:j1], float(scale), False, None)
            if causal:
                s = np.where(np.arange(j0, j1)[None, :] <= np.arange(i0, i1)[:, None], s, -np.inf)
            lse_i = lse[i0:i1]
            with np.errstate(invalid="ignore"):
                p = np.where(np.isfinite(lse_i)[:, None], np.exp(s - lse_i[:, None]), 0.0)
            dv[j0:j1] += p.T @ do[i0:i1]
            h = do[i0:i1] @ v[j0:j1].T
            ds = _score_grad(p, h, D[i0:i1])
            dq[i0:i1] += scale * (ds @ k[j0:j1])
            dk[j0:j1] += scale * (ds.T @ q[i0:i1])
    return dq, dk, dv
