"""Pins of the backward oracle (oracle/backward.py), on the CPU.

The oracle's gradients are held to things other than themselves:
* torch's float64 autograd through its own scaled_dot_product_attention (a
  library routine; "CMU 10-423 Lecture 18" notes, section 5.3 checks its
  backward the same way and reports differences around 1e-15);
* central finite differences of sum(G * O) on tiny inputs (brute force);
* closed forms: the key gradients sum to zero (softmax is unchanged when
  every key moves by the same vector), the value gradients sum to the sum of
  the upstream gradients (every row of P sums to one), D_i = G_i . O_i
  ("Infra: Flash Attention", tiled-gradient section), and a single key gives
  dV = G, dQ = dK = 0;
* the tiled recomputation from O and L equals the definition for several
  tile shapes, causal or not.
"""

import numpy as np
import pytest
import torch

import oracle


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _torch_grads(q, k, v, do, scale, causal):
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    o = torch.nn.functional.scaled_dot_product_attention(
        t[0][None, None], t[1][None, None], t[2][None, None], is_causal=causal, scale=scale
    )[0, 0]
    o.backward(torch.tensor(do, dtype=torch.float64))
    return [x.grad.numpy() for x in t]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d,scale", [(37, 16, 0.3), (64, 64, 0.125), (5, 8, 1.0)])
def test_backward_vs_torch_autograd(N, d, scale, causal):
    q, k, v, do = (_rand(10 + i, N, d) for i in range(4))
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, causal=causal)
    tq, tk, tv = _torch_grads(q, k, v, do, scale, causal)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.max(np.abs(a - b)) <= 1e-13 * max(1.0, np.max(np.abs(b)))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_vs_finite_differences(causal):
    N, d, scale = 4, 3, 0.7
    q, k, v, do = (_rand(20 + i, N, d) for i in range(4))

    def loss(q_, k_, v_):
        o, _ = oracle.attention_rows(q_, k_, v_, scale, causal=causal)
        return float((do * o).sum())

    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, causal=causal)
    eps = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.max(np.abs(num - grad)) <= 1e-7, which


@pytest.mark.parametrize("causal", [False, True])
def test_backward_closed_forms(causal):
    N, d, scale = 50, 24, 0.2
    q, k, v, do = (_rand(30 + i, N, d) for i in range(4))
    dq, dk, dv, D = oracle.attention_backward(q, k, v, do, scale, causal=causal)
    # softmax is invariant to K_j -> K_j + c for all j: the key gradients sum to 0
    assert np.max(np.abs(dk.sum(axis=0))) <= 1e-12 * np.max(np.abs(dk)) * N
    # rows of P sum to one: sum_j dV_j = sum_i G_i
    assert np.max(np.abs(dv.sum(axis=0) - do.sum(axis=0))) <= 1e-12 * N
    # D_i = sum_j P_ij (G V^T)_ij equals G_i . O_i
    o, _ = oracle.attention_rows(q, k, v, scale, causal=causal)
    assert np.max(np.abs(D - (do * o).sum(axis=1))) <= 1e-12


def test_backward_single_key():
    """One key: P = [[1]], so dV = G and dS = P (H - D) = 0."""
    q, k, v, do = (_rand(40 + i, 1, 6) for i in range(4))
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.5)
    assert np.array_equal(dv, do)
    assert np.max(np.abs(dq)) <= 1e-15 and np.max(np.abs(dk)) <= 1e-15


def test_backward_zero_upstream_gradient():
    q, k, v = (_rand(50 + i, 9, 4) for i in range(3))
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, np.zeros((9, 4)), 0.5, causal=True)
    assert not dq.any() and not dk.any() and not dv.any()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("br,bc", [(1, 1), (4, 4), (16, 8), (8, 16), (7, 5), (64, 64)])
def test_backward_tiled_equals_definition(br, bc, causal):
    N, d, scale = 45, 12, 0.4
    q, k, v, do = (_rand(60 + i, N, d) for i in range(4))
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, causal=causal)
    tq, tk, tv = oracle.attention_backward_tiled(q, k, v, do, scale, br, bc, causal=causal)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.max(np.abs(a - b)) <= 1e-13


def test_backward_ref_batched_matches_per_head():
    B, H, N, d = 2, 3, 11, 5
    Q, K, V, dO = (_rand(70 + i, B, H, N, d) for i in range(4))
    dq, dk, dv = oracle.attention_backward_ref(Q, K, V, dO, 0.3, causal=True)
    for b in range(B):
        for h in range(H):
            a = oracle.attention_backward(Q[b, h], K[b, h], V[b, h], dO[b, h], 0.3, causal=True)
            assert np.array_equal(dq[b, h], a[0]) and np.array_equal(dk[b, h], a[1]) and np.array_equal(dv[b, h], a[2])
