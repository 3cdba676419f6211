"""Pins of the float64 oracle against what the pages fix.

Every check here compares the oracle with something other than itself: a
value printed on a page (fixtures under tests/golden/, each with its
citation), a closed form, an invariant proven on a page, or an independent
library routine (torch's float64 CPU scaled_dot_product_attention,
torch.logsumexp, scipy's softmax).
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from synth import np_normal

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# (m, l, u) merge: the 49/15 worked example ("Infra: Flash Attention")
# --------------------------------------------------------------------------

def test_merge_worked_example_printed_values():
    g = gold("merge_worked_example.json")
    x = np.log(np.array(g["exp_scores"], dtype=np.float64))
    v = np.array(g["values"], dtype=np.float64)
    a = oracle.block_state(x[g["left_block"]], v[g["left_block"]])
    b = oracle.block_state(x[g["right_block"]], v[g["right_block"]])
    p = g["printed"]
    assert a[0] == pytest.approx(math.log(2), abs=1e-15)  # m_A = log 2
    assert b[0] == pytest.approx(math.log(8), abs=1e-15)  # m_B = log 8
    # the left block is rescaled by e^{log 2 - log 8} = 1/4
    assert math.exp(a[0] - max(a[0], b[0])) == pytest.approx(p["left_rescale_factor"], abs=1e-15)
    m, l, u = oracle.merge(a, b)
    assert l == pytest.approx(p["l_merged"], abs=1e-14)
    assert float(u) == pytest.approx(p["u_merged"], abs=1e-14)
    o, lse = oracle.finalize((m, l, u))
    assert float(o) == pytest.approx(p["output_numerator"] / p["output_denominator"], abs=1e-14)
    # L = log sum_j e^{x_j} ("Backward and recomputation") = log(1+2+4+8)
    assert lse == pytest.approx(math.log(15), abs=1e-14)
    # merging in the other order gives the same state
    m2, l2, u2 = oracle.merge(b, a)
    assert (m2, l2) == pytest.approx((m, l), abs=1e-15) and float(u2) == pytest.approx(float(u), abs=1e-15)
    # averaging the two block outputs is wrong (the page's warning): 5/3 and 11/3 -> 8/3
    assert abs((float(a[2]) / a[1] + float(b[2]) / b[1]) / 2 - 49 / 15) > 0.5


def test_worked_example_through_attention_and_decode():
    """The same example embedded in an attention head: query e_1, keys whose
    first coordinate is j*log 2 (so e^{score} = 1, 2, 4, 8 with scale 1) and
    values whose first coordinate is j+1."""
    g = gold("merge_worked_example.json")
    d = 8
    n = len(g["exp_scores"])
    q = np.zeros((n, d)); q[:, 0] = 1.0
    k = np.zeros((n, d)); k[:, 0] = np.log(np.array(g["exp_scores"], dtype=np.float64))
    v = np.zeros((n, d)); v[:, 0] = g["values"]; v[:, 1] = 1.0
    O, L = oracle.attention_ref(q, k, v, scale=1.0)
    assert O[0, 0] == pytest.approx(49 / 15, abs=1e-14)
    assert O[0, 1] == pytest.approx(1.0, abs=1e-14)
    assert L[0] == pytest.approx(math.log(15), abs=1e-14)
    o, lse = oracle.decode_ref(q[0], k, v, scale=1.0)
    assert o[0] == pytest.approx(49 / 15, abs=1e-14) and lse == pytest.approx(math.log(15), abs=1e-14)


def test_combine_partials_worked_example():
    """Flash-Decoding combine (airsota card, section 3, step 3) of the two
    blocks of the worked example, given as normalised partials."""
    g = gold("merge_worked_example.json")
    x = np.log(np.array(g["exp_scores"], dtype=np.float64))
    v = np.array(g["values"], dtype=np.float64)[:, None]
    parts = [oracle.block_state(x[idx], v[idx]) for idx in (g["left_block"], g["right_block"])]
    o_k = np.stack([u / l for (_, l, u) in parts])
    m_k = np.array([m for (m, _, _) in parts])
    l_k = np.array([l for (_, l, _) in parts])
    np.testing.assert_allclose(o_k[:, 0], [5 / 3, 11 / 3], atol=1e-15)
    o, lse = oracle.combine_partials(o_k, m_k, l_k)
    assert o[0] == pytest.approx(49 / 15, abs=1e-14)
    assert lse == pytest.approx(math.log(15), abs=1e-14)
    # an empty chunk (m = -inf, l = 0) gets weight 0
    o2, lse2 = oracle.combine_partials(
        np.vstack([o_k, [[123.0]]]), np.append(m_k, -np.inf), np.append(l_k, 0.0)
    )
    assert o2[0] == pytest.approx(49 / 15, abs=1e-14) and lse2 == pytest.approx(lse, abs=1e-15)
    oe, le = oracle.combine_partials(np.zeros((3, 1)), np.full(3, -np.inf), np.zeros(3))
    assert oe[0] == 0.0 and le == -np.inf


# --------------------------------------------------------------------------
# merge order-freedom ("CMU 10-423 Lecture 18", section 2.3)
# --------------------------------------------------------------------------

def _merge_all(states, order):
    if order == "left_to_right":
        acc = states[0]
        for s in states[1:]:
            acc = oracle.merge(acc, s)
        return acc
    if order == "right_to_left":
        acc = states[-1]
        for s in reversed(states[:-1]):
            acc = oracle.merge(s, acc)
        return acc
    if order == "pairwise":
        cur = list(states)
        while len(cur) > 1:
            nxt = [oracle.merge(cur[i], cur[i + 1]) for i in range(0, len(cur) - 1, 2)]
            if len(cur) % 2:
                nxt.append(cur[-1])
            cur = nxt
        return cur[0]
    if order == "shuffled":
        perm = np.random.default_rng(7).permutation(len(states))
        acc = states[perm[0]]
        for p in perm[1:]:
            acc = oracle.merge(acc, states[p])
        return acc
    raise ValueError(order)


@pytest.mark.parametrize("order", ["left_to_right", "right_to_left", "pairwise", "shuffled"])
def test_merge_order_invariance(order):
    rng = np.random.default_rng(11)
    s = rng.standard_normal(64) * 3.0
    v = rng.standard_normal((64, 16))
    states = [oracle.block_state(s[i:i + 8], v[i:i + 8]) for i in range(0, 64, 8)]
    o, lse = oracle.finalize(_merge_all(states, order))
    ref = scipy.special.softmax(s) @ v  # library softmax of the whole row
    # the lecture reports 2e-16 .. 3e-16 for all four orders
    assert np.max(np.abs(o - ref)) < 1e-14
    assert lse == pytest.approx(scipy.special.logsumexp(s), abs=1e-13)


def test_cheating_per_block_softmax_is_wrong():
    """Negative control: per-block softmax sums to the number of blocks
    (section 1.4 prints 3.000 for 12 scores in 3 blocks) and its weighted sum
    is O(1) away from softmax(s)V (section 2.3)."""
    g = gold("per_block_softmax_section14.json")
    rng = np.random.default_rng(3)
    s = rng.standard_normal(g["n_scores"]) * 2
    p = oracle.per_block_softmax(s, g["n_scores"] // g["n_blocks"])
    assert p.sum() == pytest.approx(g["printed"]["sum_of_concatenation"], abs=1e-12)
    assert scipy.special.softmax(s).sum() == pytest.approx(g["printed"]["correct_sum"], abs=1e-12)
    s64 = rng.standard_normal(64) * 3
    v = rng.standard_normal((64, 16))
    cheat = oracle.per_block_softmax(s64, 8) @ v
    assert np.max(np.abs(cheat - scipy.special.softmax(s64) @ v)) > 0.1


# --------------------------------------------------------------------------
# scalar online softmax ("CMU 10-423 Lecture 18", section 2.2, Exercise 1)
# --------------------------------------------------------------------------

def test_online_softmax_row():
    g = gold("online_row_section22.json")
    x = np.array(g["row"], dtype=np.float64)
    m, dsum = oracle.online_softmax(x)
    # the running maximum grows exactly when 3 and 6 are read
    grew = [x[j] for j in range(len(x)) if j > 0 and m[j] > m[j - 1]]
    assert grew == g["printed"]["max_increases_on_reading"]
    # Exercise 1: d_j = sum_{k<=j} e^{x_k - m_j} with m_j = max_{k<=j} x_k
    for j in range(len(x)):
        mj = x[: j + 1].max()
        assert m[j] == mj
        assert dsum[j] == pytest.approx(np.exp(x[: j + 1] - mj).sum(), rel=1e-15)
    # after the whole row: softmax = e^{x - m_N} / d_N (library softmax)
    np.testing.assert_allclose(np.exp(x - m[-1]) / dsum[-1], scipy.special.softmax(x), atol=1e-16)


# --------------------------------------------------------------------------
# the definition against independent library routines
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 8), (7, 16), (65, 32), (200, 64), (130, 128)])
def test_attention_vs_torch_sdpa(N, d, causal):
    rng = np.random.default_rng(N * 131 + d + int(causal))
    B, H = 2, 3
    Q = rng.standard_normal((B, H, N, d))
    K = rng.standard_normal((B, H, N, d))
    V = rng.standard_normal((B, H, N, d))
    scale = 1.0 / math.sqrt(d)
    O, L = oracle.attention_ref(Q, K, V, scale, causal=causal)
    tq, tk, tv = (torch.from_numpy(a) for a in (Q, K, V))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    assert np.max(np.abs(O - ref.numpy())) < 1e-12
    s = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) * scale
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    lref = torch.logsumexp(s, dim=-1).numpy()
    assert np.max(np.abs(L - lref)) < 1e-12
    # P = e^{S - L} sums to one along each row ("Backward and recomputation")
    assert np.max(np.abs(torch.exp(s - torch.from_numpy(L)[..., None]).sum(-1).numpy() - 1)) < 1e-12


def test_attention_closed_forms():
    rng = np.random.default_rng(5)
    N, d = 37, 16
    V = rng.standard_normal((N, d))
    K = rng.standard_normal((N, d))
    # constant scores (q = 0): O_i = mean of the valid V_j, L_i = log(#valid)
    Q0 = np.zeros((N, d))
    O, L = oracle.attention_ref(Q0, K, V, 0.25)
    np.testing.assert_allclose(O, np.broadcast_to(V.mean(0), O.shape), atol=1e-14)
    np.testing.assert_allclose(L, np.log(N), atol=1e-14)
    Oc, Lc = oracle.attention_ref(Q0, K, V, 0.25, causal=True)
    for i in range(N):
        np.testing.assert_allclose(Oc[i], V[: i + 1].mean(0), atol=1e-14)
        assert Lc[i] == pytest.approx(math.log(i + 1), abs=1e-14)
    # causal row 0 sees only key 0: O_0 = V_0, L_0 = S_00
    Q = rng.standard_normal((N, d))
    Oc, Lc = oracle.attention_ref(Q, K, V, 0.3, causal=True)
    np.testing.assert_allclose(Oc[0], V[0], atol=1e-15)
    assert Lc[0] == pytest.approx(0.3 * float(Q[0] @ K[0]), abs=1e-14)
    # N = 1: O = V_0
    O1, L1 = oracle.attention_ref(Q[:1], K[:1], V[:1], 0.3)
    np.testing.assert_allclose(O1[0], V[0], atol=1e-15)
    # a joint permutation of the (K, V) rows changes nothing (non-causal)
    perm = rng.permutation(N)
    Op, Lp = oracle.attention_ref(Q, K[perm], V[perm], 0.3)
    On, Ln = oracle.attention_ref(Q, K, V, 0.3)
    np.testing.assert_allclose(Op, On, atol=1e-14)
    np.testing.assert_allclose(Lp, Ln, atol=1e-14)
    # a shift of every score of a row by c leaves O unchanged and moves L by c:
    # adding c * q_i / (scale |q_i|^2) to every key
    c = 5.0
    shift = (c / (0.3 * (Q * Q).sum(1)))[:, None] * Q
    for i in (0, 10, 36):
        Os, Ls = oracle.attention_rows(Q[i:i + 1], K + shift[i], V, 0.3)
        np.testing.assert_allclose(Os[0], On[i], atol=1e-12)
        assert Ls[0] == pytest.approx(Ln[i] + c, abs=1e-12)


def test_attention_rows_matches_sdpa_on_selected_rows():
    rng = np.random.default_rng(9)
    N, d = 300, 32
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    rows = np.array([0, 1, 63, 64, 150, 299])
    O, L = oracle.attention_rows(Q[rows], K, V, 0.2, causal=True, q_pos=rows)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a)[None] for a in (Q, K, V)), is_causal=True, scale=0.2
    )[0].numpy()
    assert np.max(np.abs(O - ref[rows])) < 1e-12


def test_decode_ref_against_sdpa_and_empty_cache():
    rng = np.random.default_rng(21)
    Lk, d = 1000, 64
    q = rng.standard_normal(d)
    K = rng.standard_normal((Lk, d)) * 2
    V = rng.standard_normal((Lk, d)) * 2
    o, lse = oracle.decode_ref(q, K, V, 1 / 8)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(K)[None], torch.from_numpy(V)[None], scale=1 / 8
    )[0, 0].numpy()
    assert np.max(np.abs(o - ref)) < 1e-12
    assert lse == pytest.approx(float(torch.logsumexp(torch.from_numpy(K @ q) / 8, 0)), abs=1e-12)
    oe, le = oracle.decode_ref(q, K[:0], V[:0], 1 / 8)
    assert np.all(oe == 0) and le == -np.inf


@pytest.mark.parametrize("chunk", [1, 7, 64, 333, 1000, 4096])
def test_split_and_combine_equals_decode(chunk):
    """Flash-Decoding (airsota card, section 3): per-chunk partials merged by
    the log-sum-exp reduction equal the single-pass result, for any chunking
    including empty trailing chunks."""
    rng = np.random.default_rng(chunk)
    Lk, d = 1000, 32
    q = rng.standard_normal(d)
    K = rng.standard_normal((Lk, d))
    V = rng.standard_normal((Lk, d))
    o_ref, lse_ref = oracle.decode_ref(q, K, V, 0.25)
    parts_o, parts_m, parts_l = [], [], []
    for c0 in range(0, max(Lk, chunk * 3), chunk):
        m, l, u = oracle.block_state((K[c0:c0 + chunk] @ q) * 0.25, V[c0:c0 + chunk])
        parts_o.append(u / l if l > 0 else np.zeros(d))
        parts_m.append(m)
        parts_l.append(l)
    o, lse = oracle.combine_partials(parts_o, parts_m, parts_l)
    assert np.max(np.abs(o - o_ref)) < 1e-13
    assert lse == pytest.approx(lse_ref, abs=1e-13)


# --------------------------------------------------------------------------
# tiled Algorithm 1 against the definition, and the traffic model
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Br,Bc", [(1, 1), (3, 4), (4, 3), (16, 16), (64, 16), (16, 64), (256, 256), (100, 37)])
def test_tiled_equals_full(Br, Bc, causal):
    """'CMU 10-423 Lecture 18', section 3.3: at N = 256, d = 32 in float64 the
    tiled result differs from full attention only by rounding."""
    rng = np.random.default_rng(Br * 1000 + Bc)
    N, d = 256, 32
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    O, L = oracle.tiled_ref(Q, K, V, Br, Bc, 1 / math.sqrt(d), causal=causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a)[None] for a in (Q, K, V)), is_causal=causal, scale=1 / math.sqrt(d)
    )[0].numpy()
    assert np.max(np.abs(O - ref)) < 1e-13
    Of, Lf = oracle.attention_ref(Q, K, V, 1 / math.sqrt(d), causal=causal)
    assert np.max(np.abs(L - Lf)) < 1e-13


def test_tiled_masked_row_guard():
    """A tile in which some rows have no valid key must leave those rows'
    state untouched (no -inf - (-inf)); with B_r = 8 > B_c = 2, causal, the
    first tiles of every query tile fully mask most rows."""
    rng = np.random.default_rng(1)
    N, d = 24, 4
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    O, L = oracle.tiled_ref(Q, K, V, 8, 2, 0.5, causal=True)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a)[None] for a in (Q, K, V)), is_causal=True, scale=0.5
    )[0].numpy()
    assert np.max(np.abs(O - ref)) < 1e-13


def test_io_counts_exercise3():
    g = gold("io_counts_exercise3.json")
    N, d, Br = g["N"], g["d"], g["Br"]
    p = g["printed"]
    assert oracle.io_standard(N, d) == p["standard_forward_elements"]
    assert oracle.io_fa2(N, d, Br) == p["fa2_forward_elements"] == sum(p["fa2_terms"])
    assert oracle.io_standard(N, d) / oracle.io_fa2(N, d, Br) == pytest.approx(p["saving_ratio"], abs=0.005)
    assert 2 * Br / d == p["saving_ratio"]
    # the tiled loop, run at this exact size, moves exactly that many elements
    rng = np.random.default_rng(0)
    Q, K, V = (rng.standard_normal((N, d)).astype(np.float32) for _ in range(3))
    _, _, cnt = oracle.tiled_ref(Q, K, V, Br, 512, 1 / math.sqrt(d), count=True)
    assert cnt["reads"] + cnt["writes"] == p["fa2_forward_elements"]
    assert cnt["tiles"] == (N // Br) * (N // 512)


def test_causal_tiles_exercise4():
    g = gold("causal_tiles_exercise4.json")
    T, N, blk = g["T"], g["N"], g["block"]
    rng = np.random.default_rng(0)
    Q, K, V = (rng.standard_normal((N, 4)) for _ in range(3))
    _, _, cnt = oracle.tiled_ref(Q, K, V, blk, blk, 0.5, causal=True, count=True)
    assert cnt["tiles"] == oracle.causal_tile_count(T)
    num, den = g["printed"]["flop_ratio_fraction"]
    assert cnt["tiles"] / T ** 2 == pytest.approx(num / den, abs=0)
    assert round(cnt["tiles"] / T ** 2, 3) == g["printed"]["flop_ratio"]


def test_io_savings_section41():
    g = gold("io_savings_section41.json")
    d, M = g["d"], g["M"]
    p = g["printed"]
    # FA-1 block rule of the lecture: B_c = ceil(M / 4d), B_r = min(B_c, d)
    assert -(-M // (4 * d)) == g["fa1_Bc"] and min(-(-M // (4 * d)), d) == g["fa1_Br"]
    N = 1 << 20
    assert round(oracle.io_standard(N, d) / oracle.io_fa1_main(N, d, M), 1) == p["fa1_saving_limit"]
    assert round(oracle.io_standard(N, d) / oracle.io_fa2(N, d, g["fa2_Br"]), 1) == p["fa2_saving_limit"]
    # section 4.2: the FA-1 order moves fewer elements than 4N^2 iff M > 3d^2
    thr = p["fa1_needs_M_above"]
    assert 3 * d * d == thr
    assert oracle.io_fa1_main(N, d, thr + 64) < 4 * N * N < oracle.io_fa1_main(N, d, thr - 64)
    # on-chip peak of the FA-1 loop: K_j, V_j, Q_i, O_i, S_ij and l, m
    Bc, Br = g["fa1_Bc"], g["fa1_Br"]
    peak = 2 * Bc * d + 2 * Br * d + Br * Bc + 2 * Br
    assert peak / M <= p["onchip_peak_fraction_at_most"]


def test_bf16_inputs_are_exact_in_float64():
    x = np_normal(3, (1000,), dtype="bf16")
    bits = x.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    ref = torch.from_numpy(np.random.default_rng(3).standard_normal(1000, dtype=np.float32)).to(torch.bfloat16)
    np.testing.assert_array_equal(x, ref.float().numpy())


def test_attention_dev_rows_brute_force_and_closed_forms():
    """attention_dev_rows against its definition written as plain loops on a
    tiny input, and closed forms: one valid key (causal row 0) leaves no
    spread; two keys with equal scores spread by |v1 - v2| / 2."""
    rng = np.random.default_rng(31)
    N, d, dv = 6, 4, 3
    Q, K, V = rng.standard_normal((N, d)), rng.standard_normal((N, d)), rng.standard_normal((N, dv))
    for causal in (False, True):
        dev, am = oracle.attention_dev_rows(Q, K, V, 0.7, causal=causal)
        for i in range(N):
            keys = [j for j in range(N) if not causal or j <= i]
            s = [0.7 * sum(Q[i, t] * K[j, t] for t in range(d)) for j in keys]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            tot = sum(e)
            p = [x / tot for x in e]
            for c in range(dv):
                o = sum(pj * V[j, c] for pj, j in zip(p, keys))
                assert dev[i, c] == pytest.approx(sum(pj * abs(V[j, c] - o) for pj, j in zip(p, keys)), abs=1e-13)
                assert am[i, c] == pytest.approx(sum(pj * abs(V[j, c]) for pj, j in zip(p, keys)), abs=1e-13)
        if causal:
            np.testing.assert_allclose(dev[0], 0.0, atol=1e-15)
            np.testing.assert_allclose(am[0], np.abs(V[0]), atol=1e-15)
    v2 = np.array([[1.0, -2.0], [3.0, 5.0]])
    dev, am = oracle.attention_dev_rows(np.zeros((1, 4)), rng.standard_normal((2, 4)), v2, 1.0)
    np.testing.assert_allclose(dev[0], [1.0, 3.5], atol=1e-15)
    np.testing.assert_allclose(am[0], [2.0, 3.5], atol=1e-15)


def test_attention_dev_rows_bounds_rounded_probabilities():
    """The use it is made for: perturbing every probability by a relative
    amount of at most delta and renormalising moves O by at most
    delta / (1 - delta) * dev."""
    rng = np.random.default_rng(32)
    N, d = 200, 16
    Q, K, V = (rng.standard_normal((N, d)) * 3 for _ in range(3))
    O, L = oracle.attention_ref(Q, K, V, 0.4)
    dev, _ = oracle.attention_dev_rows(Q, K, V, 0.4)
    P = np.exp(Q @ K.T * 0.4 - L[:, None])
    delta = 2.0 ** -8
    worst = 0.0
    for trial in range(20):
        Pp = P * (1 + delta * rng.choice([-1.0, 1.0], size=P.shape) * rng.uniform(0.5, 1.0, size=P.shape))
        Op = (Pp @ V) / Pp.sum(1, keepdims=True)
        worst = max(worst, float(np.max(np.abs(Op - O) / (delta / (1 - delta) * dev + 1e-300))))
    assert worst <= 1.0
    assert worst > 0.05  # the bound is not vacuous
