"""Online softmax, the (m, l, u) block state, its merge, and the
Flash-Decoding log-sum-exp combine, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* Scalar online softmax: "CMU 10-423 Lecture 18" notes, section 2.1 (online
  form) and Exercise 1 (the recurrence d_j = d_{j-1} e^{m_{j-1}-m_j} +
  e^{x_j - m_j} and its induction).
* Block state and merge: "Infra: Flash Attention", section "Online softmax and
  state merging" (merging block states: m = max(m_A, m_B), alpha =
  e^{m_A - m}, beta = e^{m_B - m}, l = alpha l_A + beta l_B; accumulating the
  weighted sum: u = alpha u_A + beta u_B, O = u / l); the same (m, l, o)
  merge in the lecture notes, section 2.3 and Exercise 2.
* Combine of split partials: the airsota Flash-Decoding card, section 3,
  step 3 (log-sum-exp reduction: m_final = max_k m^(k), l_final =
  sum_k l^(k) e^{m^(k) - m_final}, O = sum_k O^(k) l^(k) e^{m^(k) - m_final}
  / l_final).  The card's typeset minus signs were extracted as dashes; they
  are read as minus signs.

An empty block (no scores, or all scores -inf) has the state (-inf, 0, 0).
Merging with it changes nothing; its factor e^{-inf - m} is taken as 0
without forming -inf - (-inf) ("Infra: Flash Attention", section "Notation and
boundary conditions").
"""

import numpy as np


def _factor(m_part, m_new):
    """e^{m_part - m_new}, with an empty part (m_part = -inf) giving 0."""
    if m_part == -np.inf:
        return 0.0
    return float(np.exp(m_part - m_new))


def online_softmax(x):
    """Scalar online softmax over one row x_1..x_N.

    Returns (m, dsum): arrays of the running maximum m_j and the running
    normaliser d_j after reading element j (1-based j <-> index j-1)."""
    x = np.asarray(x, dtype=np.float64)
    m_prev, d_prev = -np.inf, 0.0
    ms, ds = [], []
    for xj in x:
        m_j = max(m_prev, float(xj))
        d_j = d_prev * _factor(m_prev, m_j) + float(np.exp(xj - m_j))
        ms.append(m_j)
        ds.append(d_j)
        m_prev, d_prev = m_j, d_j
    return np.array(ms), np.array(ds)


def block_state(s, v):
    """State of one block of scores s [n] with values v [n, dv] (or [n]):
    m = max s, l = sum e^{s - m}, u = sum e^{s - m} v_j."""
    s = np.asarray(s, dtype=np.float64).reshape(-1)
    v = np.asarray(v, dtype=np.float64)
    vshape = v.shape[1:]
    if s.size == 0 or not np.isfinite(s.max()):
        return (-np.inf, 0.0, np.zeros(vshape))
    m = float(s.max())
    w = np.exp(s - m)
    return (m, float(w.sum()), np.tensordot(w, v, axes=(0, 0)))


def merge(a, b):
    """Merge two states (m, l, u) onto the common base m = max(m_a, m_b)."""
    m_a, l_a, u_a = a
    m_b, l_b, u_b = b
    m = max(m_a, m_b)
    if m == -np.inf:
        return (-np.inf, 0.0, np.zeros_like(np.asarray(u_a, dtype=np.float64)))
    alpha = _factor(m_a, m)
    beta = _factor(m_b, m)
    return (
        m,
        alpha * l_a + beta * l_b,
        alpha * np.asarray(u_a, dtype=np.float64) + beta * np.asarray(u_b, dtype=np.float64),
    )


def finalize(state):
    """O = u / l and L = m + log l; an empty state gives (0, -inf)."""
    m, l, u = state
    u = np.asarray(u, dtype=np.float64)
    if l == 0.0:
        return np.zeros_like(u), -np.inf
    return u / l, m + float(np.log(l))


def combine_partials(o_parts, m_parts, l_parts):
    """Flash-Decoding reduction of K partials.

    o_parts [K, dv]: normalised partial outputs O^(k); m_parts [K], l_parts
    [K]: each chunk's maximum and normaliser.  Returns (O [dv], lse) with
    lse = m_final + log l_final.  Partials with l^(k) = 0 (empty chunks,
    m^(k) = -inf) get weight 0; if every chunk is empty the result is
    (0, -inf)."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    m_parts = np.asarray(m_parts, dtype=np.float64)
    l_parts = np.asarray(l_parts, dtype=np.float64)
    m_final = m_parts.max() if m_parts.size else -np.inf
    if m_final == -np.inf:
        return np.zeros(o_parts.shape[1:]), -np.inf
    scaled = np.array([l_k * _factor(m_k, m_final) for m_k, l_k in zip(m_parts, l_parts)])
    l_final = scaled.sum()
    o = np.tensordot(scaled / l_final, o_parts, axes=(0, 0))
    return o, float(m_final + np.log(l_final))


def per_block_softmax(s, block):
    """The 'cheating' per-block softmax: each block of `block` scores is
    normalised on its own and the results are concatenated ("CMU 10-423
    Lecture 18", sections 1.4 and 2.3).  Not exact; used as a negative
    control only."""
    s = np.asarray(s, dtype=np.float64).reshape(-1)
    out = np.empty_like(s)
    for b0 in range(0, s.size, block):
        seg = s[b0:b0 + block]
        e = np.exp(seg - seg.max())
        out[b0:b0 + block] = e / e.sum()
    return out
