"""Planted mistakes in the oracle (on the CPU) must fail at least one pin.

Each case patches one plausible error into the oracle -- a wrong sign, a
dropped term, a transposed operand, the wrong log base -- and checks that the
pin tests of test_oracle_pins.py reject it.
"""

import numpy as np
import pytest

import oracle
import oracle.attention as att
import oracle.online as onl
import oracle.tiled as til
import tests.test_oracle_pins as pins


def _fails(fn, *args, **kw):
    try:
        fn(*args, **kw)
    except AssertionError:
        return True
    return False


def test_inverted_rescale_factor_is_caught(monkeypatch):
    monkeypatch.setattr(onl, "_factor", lambda m_part, m_new: 0.0 if m_part == -np.inf else float(np.exp(m_new - m_part)))
    assert _fails(pins.test_merge_worked_example_printed_values)
    assert _fails(pins.test_combine_partials_worked_example)


def test_merge_forgetting_to_rescale_u_is_caught(monkeypatch):
    orig = onl.merge

    def bad_merge(a, b):
        m, l, _ = orig(a, b)
        return (m, l, np.asarray(a[2], dtype=np.float64) + np.asarray(b[2], dtype=np.float64))

    monkeypatch.setattr(onl, "merge", bad_merge)
    monkeypatch.setattr(oracle, "merge", bad_merge)
    assert _fails(pins.test_merge_worked_example_printed_values)
    assert _fails(pins.test_merge_order_invariance, "pairwise")


def test_dropped_scale_is_caught(monkeypatch):
    orig = att._rows_of_attention
    monkeypatch.setattr(att, "_rows_of_attention", lambda q, k, v, scale, causal, q_pos: orig(q, k, v, 1.0, causal, q_pos))
    assert _fails(pins.test_attention_vs_torch_sdpa, 65, 32, False)


def test_log2_lse_is_caught(monkeypatch):
    orig = att._rows_of_attention

    def log2_rows(q, k, v, scale, causal, q_pos):
        o, lse = orig(q, k, v, scale, causal, q_pos)
        return o, lse / np.log(2.0)

    monkeypatch.setattr(att, "_rows_of_attention", log2_rows)
    assert _fails(pins.test_worked_example_through_attention_and_decode)


def test_lse_without_max_is_caught(monkeypatch):
    orig = att._rows_of_attention

    def no_max(q, k, v, scale, causal, q_pos):
        o, lse = orig(q, k, v, scale, causal, q_pos)
        s = (q @ k.T) * scale
        if causal:
            s = np.where(np.arange(k.shape[0])[None, :] <= q_pos[:, None], s, -np.inf)
        return o, lse - s.max(axis=1)

    monkeypatch.setattr(att, "_rows_of_attention", no_max)
    assert _fails(pins.test_worked_example_through_attention_and_decode)


def test_transposed_scores_are_caught(monkeypatch):
    """softmax over the query axis instead of the key axis."""

    def transposed(q, k, v, scale, causal, q_pos):
        s = (k @ q.T).T * scale
        s = s - s.max(axis=0, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=0, keepdims=True)
        return p @ v, np.log(np.exp(s).sum(axis=1))

    monkeypatch.setattr(att, "_rows_of_attention", transposed)
    assert _fails(pins.test_attention_vs_torch_sdpa, 7, 16, False)


def test_reversed_causal_mask_is_caught(monkeypatch):
    orig = att._rows_of_attention

    def anti_causal(q, k, v, scale, causal, q_pos):
        if not causal:
            return orig(q, k, v, scale, causal, q_pos)
        n = k.shape[0]
        # keeps keys j >= i instead of j <= i
        return orig(q, k[::-1], v[::-1], scale, True, n - 1 - q_pos)

    monkeypatch.setattr(att, "_rows_of_attention", anti_causal)
    assert _fails(pins.test_attention_closed_forms)
    assert _fails(pins.test_attention_vs_torch_sdpa, 65, 32, True)


def test_tiled_without_alpha_is_caught(monkeypatch):
    real_exp = np.exp

    class FakeNp:
        def __getattr__(self, name):
            return getattr(np, name)

        @staticmethod
        def exp(x):
            return real_exp(x)

        @staticmethod
        def where(cond, a, b):
            # alpha = where(finite(m), exp(m - m'), 0) replaced by 1
            if np.ndim(b) == 0 and b == 0.0 and np.ndim(a) == 1 and np.all(np.asarray(a) <= 1.0):
                return np.ones_like(np.asarray(a, dtype=np.float64))
            return np.where(cond, a, b)

    monkeypatch.setattr(til, "np", FakeNp())
    assert _fails(pins.test_tiled_equals_full, 16, 16, False)


def test_tiled_visiting_future_tiles_is_caught(monkeypatch):
    orig = til.tiled_ref

    def no_skip(Q, K, V, Br, Bc, scale, causal=False, count=False):
        out = orig(Q, K, V, Br, Bc, scale, causal=causal, count=count)
        if count and causal:
            n = -(-np.asarray(Q).shape[0] // Br) * -(-np.asarray(K).shape[0] // Bc)
            out[2]["tiles"] = n
        return out

    monkeypatch.setattr(oracle, "tiled_ref", no_skip)
    assert _fails(pins.test_causal_tiles_exercise4)


def test_io_formula_off_by_one_term_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "io_fa2", lambda N, d, Br: 2 * N * d * (-(-N // Br)) + 2 * N * d)
    assert _fails(pins.test_io_counts_exercise3)


# ---- paged-KV decode oracle ("CMU 10-423 Lecture 18", section 7.3)

import oracle.paged as pgd
import tests.test_oracle_paged as ppins


def test_gather_ignoring_the_block_table_is_caught(monkeypatch):
    def logical_gather(pool, table_row, length, block_size):
        nb = pgd.blocks_of(length, block_size)
        H, d = pool.shape[1], pool.shape[3]
        if nb == 0:
            return np.zeros((H, 0, d))
        parts = [np.asarray(pool[i], dtype=np.float64) for i in range(nb)]  # logical index, no table
        return np.concatenate(parts, axis=1)[:, :length]

    monkeypatch.setattr(pgd, "gather_paged", logical_gather)
    monkeypatch.setattr(oracle, "gather_paged", logical_gather)
    assert _fails(ppins.test_worked_example_section73)
    assert _fails(ppins.test_gather_is_exact_and_blockwise_matches_plain, 4, 17)


def test_reading_the_whole_last_block_is_caught(monkeypatch):
    def untrimmed(pool, table_row, length, block_size):
        nb = pgd.blocks_of(length, block_size)
        H, d = pool.shape[1], pool.shape[3]
        if nb == 0:
            return np.zeros((H, 0, d))
        return np.concatenate([np.asarray(pool[int(table_row[i])], dtype=np.float64) for i in range(nb)], axis=1)

    monkeypatch.setattr(pgd, "gather_paged", untrimmed)
    assert _fails(ppins.test_slots_past_the_end_are_never_read)


def test_blockwise_without_rescaling_is_caught(monkeypatch):
    def naive_merge(a, b):  # adds states without moving them to a common base
        return (max(a[0], b[0]), a[1] + b[1], np.asarray(a[2], dtype=np.float64) + np.asarray(b[2], dtype=np.float64))

    monkeypatch.setattr(pgd, "merge", naive_merge)
    assert _fails(ppins.test_worked_example_section73)


# --------------------------------------------------------------------------
# backward oracle
# --------------------------------------------------------------------------

import oracle.backward as bwd  # noqa: E402
import tests.test_oracle_backward as bpins  # noqa: E402


def test_backward_D_without_P_is_caught(monkeypatch):
    monkeypatch.setattr(bwd, "_row_D", lambda p, h: h.sum(axis=1))
    assert _fails(bpins.test_backward_vs_torch_autograd, 37, 16, 0.3, False)
    assert _fails(bpins.test_backward_closed_forms, False)


def test_backward_dropped_D_is_caught(monkeypatch):
    monkeypatch.setattr(bwd, "_score_grad", lambda p, h, D: p * h)
    assert _fails(bpins.test_backward_vs_finite_differences, False)


def test_backward_flipped_score_gradient_sign_is_caught(monkeypatch):
    monkeypatch.setattr(bwd, "_score_grad", lambda p, h, D: p * (D[:, None] - h))
    assert _fails(bpins.test_backward_vs_torch_autograd, 64, 64, 0.125, True)


def test_backward_unnormalised_probabilities_are_caught(monkeypatch):
    monkeypatch.setattr(bwd, "_softmax_rows", lambda s: np.exp(s - s.max(axis=1)[:, None]))
    assert _fails(bpins.test_backward_vs_torch_autograd, 37, 16, 0.3, True)


def test_backward_tiled_with_log2_lse_is_caught(monkeypatch):
    orig = bwd.attention_backward_tiled

    def bad(q, k, v, do, scale, br, bc, causal=False, o=None, lse=None):
        o_, l_ = oracle.attention_rows(q, k, v, scale, causal=causal)
        return orig(q, k, v, do, scale, br, bc, causal=causal, o=o_, lse=l_ / np.log(2.0))

    monkeypatch.setattr(oracle, "attention_backward_tiled", bad)
    assert _fails(bpins.test_backward_tiled_equals_definition, 16, 8, False)


def test_backward_dropped_causal_mask_is_caught(monkeypatch):
    orig_scores = bwd._masked_scores
    monkeypatch.setattr(bwd, "_masked_scores", lambda q, k, scale, causal, q_pos: orig_scores(q, k, scale, False, q_pos))
    assert _fails(bpins.test_backward_vs_torch_autograd, 37, 16, 0.3, True)


def test_dev_around_zero_instead_of_o_is_caught(monkeypatch):
    orig = att.attention_dev_rows

    def around_zero(q, k, v, scale, causal=False, q_pos=None):
        dev, am = orig(q, k, v, scale, causal, q_pos)
        return am, am

    monkeypatch.setattr(att, "attention_dev_rows", around_zero)
    monkeypatch.setattr(oracle, "attention_dev_rows", around_zero)
    assert _fails(pins.test_attention_dev_rows_brute_force_and_closed_forms)
