"""Plain definition of scaled dot-product attention, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, per head ("Infra: Flash Attention", section "Attention and
scope"; the per-row log-sum-exp from section "Backward and recomputation"):

    S = Q K^T * scale                      (scale = 1/sqrt(d) on the page)
    causal: S[i, j] = -inf for key j later than query i
    m_i = max_j S_ij
    l_i = sum_j exp(S_ij - m_i)            (stable normalisation,
                                            section "Online softmax and state
                                            merging / stable normalisation")
    O_i = sum_j exp(S_ij - m_i) V_j / l_i
    L_i = m_i + log(l_i)  = log sum_j exp(S_ij)   (natural logarithm)

attention_dev_rows gives, from the same definition, the P-weighted spread of
V around O that bounds the effect of rounding P before the product with V.

This is the definition, not the tiled algorithm: the whole row of scores is
formed (a block of rows at a time only to bound memory) and reduced with
numpy.  Inputs are upcast to float64 exactly (bf16 and fp32 values are exactly
representable in float64).

A row with no valid key at all is left open by the page ("the operator must
define the output", section "Notation and boundary conditions"); the reading
taken here is O_i = 0 and L_i = -inf.
"""

import numpy as np

_ROW_BLOCK_ELEMS = 1 << 23  # at most 8M float64 scores (64 MiB) per row block


def _rows_of_attention(q, k, v, scale, causal, q_pos):
    """Rows of one head: q [R, d], k [Nk, d], v [Nk, dv], q_pos [R] absolute
    query positions (used only when causal).  Returns (O [R, dv], L [R])."""
    s = (q @ k.T) * scale  # [R, Nk]
    if causal:
        key_pos = np.arange(k.shape[0])
        s = np.where(key_pos[None, :] <= q_pos[:, None], s, -np.inf)
    m = s.max(axis=1)  # [R]
    valid = np.isfinite(m)
    m_safe = np.where(valid, m, 0.0)
    p = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 for masked keys
    l = p.sum(axis=1)
    o_num = p @ v
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(valid[:, None], o_num / np.where(valid, l, 1.0)[:, None], 0.0)
        lse = np.where(valid, m_safe + np.log(np.where(valid, l, 1.0)), -np.inf)
    return o, lse


def attention_rows(q, k, v, scale, causal=False, q_pos=None):
    """Selected query rows of one head.

    q: [R, d] query rows; k: [Nk, d]; v: [Nk, dv]; q_pos: absolute positions
    of the R rows in the sequence (default 0..R-1).  Causal keeps key j for
    query i iff j <= q_pos[i] (top-left alignment, square attention).
    Returns float64 (O [R, dv], L [R]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q_pos is None:
        q_pos = np.arange(q.shape[0])
    q_pos = np.asarray(q_pos, dtype=np.int64)
    R = q.shape[0]
    o = np.empty((R, v.shape[1]), dtype=np.float64)
    lse = np.empty((R,), dtype=np.float64)
    rb = max(1, _ROW_BLOCK_ELEMS // max(1, k.shape[0]))
    for r0 in range(0, R, rb):
        r1 = min(R, r0 + rb)
        o[r0:r1], lse[r0:r1] = _rows_of_attention(
            q[r0:r1], k, v, float(scale), causal, q_pos[r0:r1]
        )
    return o, lse


def attention_ref(Q, K, V, scale, causal=False):
    """Full attention over arrays shaped [..., N, d] (any leading batch/head
    dims).  Returns float64 (O [..., N, d], L [..., N])."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    lead = Q.shape[:-2]
    N, d = Q.shape[-2:]
    Qf = Q.reshape(-1, N, d)
    Kf = K.reshape(-1, K.shape[-2], K.shape[-1])
    Vf = V.reshape(-1, V.shape[-2], V.shape[-1])
    O = np.empty(Qf.shape[:-1] + (Vf.shape[-1],), dtype=np.float64)
    L = np.empty(Qf.shape[:-1], dtype=np.float64)
    for s in range(Qf.shape[0]):
        O[s], L[s] = attention_rows(Qf[s], Kf[s], Vf[s], scale, causal)
    return O.reshape(lead + (N, Vf.shape[-1])), L.reshape(lead + (N,))


def attention_dev_rows(q, k, v, scale, causal=False, q_pos=None):
    """Per selected row i and value dimension e, with P the exact attention
    probabilities of the definition and O = P V:

        dev[i, e]    = sum_j P_ij |V_je - O_ie|   (P-weighted mean absolute
                                                   deviation of V around O)
        absmean[i, e] = sum_j P_ij |V_je|

    These bound how far O moves when every probability is perturbed by a
    relative amount of at most delta and the result is renormalised by the
    perturbed weights: |O' - O| <= delta / (1 - delta) * dev.  That is the
    effect of rounding the probabilities to a narrower format before the
    product with V (the probability matrix W of "Infra: Flash Attention",
    Algorithm 1, entering U = alpha U + W V).  Arguments as attention_rows.
    Returns float64 (dev [R, dv], absmean [R, dv]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q_pos is None:
        q_pos = np.arange(q.shape[0])
    q_pos = np.asarray(q_pos, dtype=np.int64)
    o, lse = attention_rows(q, k, v, scale, causal=causal, q_pos=q_pos)
    R, dv = o.shape
    dev = np.zeros((R, dv), dtype=np.float64)
    absmean = np.zeros((R, dv), dtype=np.float64)
    rb = max(1, (1 << 20) // max(1, k.shape[0] * dv // 64))
    for r0 in range(0, R, rb):
        r1 = min(R, r0 + rb)
        s = (q[r0:r1] @ k.T) * float(scale)
        if causal:
            s = np.where(np.arange(k.shape[0])[None, :] <= q_pos[r0:r1, None], s, -np.inf)
        ok = np.isfinite(lse[r0:r1])
        p = np.where(ok[:, None], np.exp(s - np.where(ok, lse[r0:r1], 0.0)[:, None]), 0.0)
        for e in range(dv):
            dev[r0:r1, e] = np.sum(p * np.abs(v[None, :, e] - o[r0:r1, e, None]), axis=1)
        absmean[r0:r1] = p @ np.abs(v)
    return dev, absmean


def decode_ref(q, K, V, scale):
    """Single-query decode ("Infra: Flash Attention", section "Prefill and
    decode": one query against the whole KV cache of length L, no mask; the
    airsota card, section 3: N_q = 1 against a cache of length L).

    q: [d]; K: [L, d]; V: [L, dv].  Returns float64 (o [dv], lse scalar).
    L = 0 (empty cache) gives o = 0, lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64).reshape(1, -1)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros((V.shape[1],), dtype=np.float64), -np.inf
    o, lse = attention_rows(q, K, V, scale, causal=False)
    return o[0], float(lse[0])
