"""CPU checks of the comparison helpers the GPU parity tests use
(tests/parity_util.py): bf16 rounding and spacing, the per-element bar, and
the two diagnostics."""

import numpy as np
import pytest
import torch

from tests.parity_util import BF16_O, Cmp, bf16_rne64, bf16_spacing, o_bar_bf16, rounded_w_bound


def test_bf16_rne64_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-3, 4, 100000),
                        # ties: 8 significant bits plus exactly one half
                        (np.arange(128, 256) + 0.5) / 128.0, -(np.arange(128, 256) + 0.5) * 4.0])
    x32 = x.astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(bf16_rne64(x32.astype(np.float64)), want)


def test_bf16_rne64_rounds_from_float64_directly():
    # 1 + 2^-8 + 2^-30 is just above the tie between 1 and 1 + 2^-7; rounding
    # through fp32 first would drop the 2^-30 and tie to 1 (even)
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert bf16_rne64(np.array([x]))[0] == 1.0 + 2.0 ** -7
    assert bf16_rne64(np.array([1.0 + 2.0 ** -8]))[0] == 1.0


def test_spacing_and_bar():
    assert bf16_spacing(np.array([1.0]))[0] == 2.0 ** -7
    assert bf16_spacing(np.array([1.999]))[0] == 2.0 ** -7
    assert bf16_spacing(np.array([-7.99]))[0] == 2.0 ** -5
    assert bf16_spacing(np.array([8.0]))[0] == 2.0 ** -4
    assert bf16_spacing(np.array([0.0]))[0] == 0.0
    bar = o_bar_bf16(np.array([0.0, 3.0, -7.99, 8.0, 17.0, -40.0]))
    assert np.array_equal(bar, [BF16_O, BF16_O, BF16_O, 2.0 ** -4, 2.0 ** -3, 2.0 ** -2])
    # half a spacing stays inside 2e-2 below |O| = 8 and does not from 8 on
    assert 0.5 * bf16_spacing(np.array([7.99]))[0] < BF16_O < 0.5 * bf16_spacing(np.array([8.0]))[0]


def test_cmp_diagnostics():
    ref = np.array([1.0 + 2.0 ** -9, 5.3, 12.7])
    c = Cmp()
    c.add_o(bf16_rne64(ref), ref)
    assert c.d_rne == 0.0 and c.excess <= 0.0 and c.ok()
    # one spacing off the rounded value: a neighbour
    c = Cmp()
    got = bf16_rne64(ref) + bf16_spacing(ref)
    c.add_o(got, ref)
    assert np.allclose(c.d_rne, bf16_spacing(ref).max()) and c.excess > 0.0
    # 12.7 off by 0.06 passes (bar 1/16), 5.3 off by 0.021 fails (bar 2e-2)
    c = Cmp()
    c.add_o(np.array([12.76]), np.array([12.7]))
    assert c.ok()
    c.add_o(np.array([5.321]), np.array([5.3]))
    assert not c.ok()


def test_cmp_l_and_empty_rows():
    c = Cmp()
    c.add_l(np.array([-np.inf, 1.0]), np.array([-np.inf, 1.001]))
    assert c.dL == pytest.approx(1e-3) and c.ok()
    with pytest.raises(AssertionError):
        c.add_l(np.array([-np.inf]), np.array([0.0]))
    c = Cmp(bf16=False)
    c.add_o(np.array([1.0 + 2e-5]), np.array([1.0]))
    assert not c.ok()


def test_rounded_w_bound_covers_an_emulated_kernel():
    """An emulation of the kernel's arithmetic in numpy -- fp32 weights
    relative to a base below the row maximum (as conditional rescaling
    leaves it), rounded to bf16 for the product, O normalised by the fp32
    sum, bf16 output -- stays within the bound on peaked rows, where the flat
    2e-2 bar does not hold."""
    import oracle

    rng = np.random.default_rng(3)
    N, d = 300, 64
    Q, K, V = (bf16_rne64(rng.standard_normal((N, d)) * 4) for _ in range(3))
    O, L = oracle.attention_ref(Q, K, V, 0.05)
    _, am = oracle.attention_dev_rows(Q, K, V, 0.05)
    s = Q @ K.T * 0.05
    base = s.max(1, keepdims=True) - rng.uniform(0, 8 * np.log(2), size=(N, 1))
    w = np.exp(s - base).astype(np.float32).astype(np.float64)
    wb = bf16_rne64(w)
    o_k = bf16_rne64((wb @ V) / w.sum(1, keepdims=True))
    bound = rounded_w_bound(O, am, N)
    assert np.all(np.abs(o_k - O) <= bound)
    assert np.max(np.abs(o_k - O)) > BF16_O  # the flat bar would not hold here


def test_excess_of_a_power_of_two_output():
    """-4.0127 rounds to -4.0 (spacing 2^-5 in [4, 8)): the stored -4.0 is the
    correctly rounded value, so it shows no kernel error."""
    c = Cmp()
    c.add_o(np.array([-4.0]), np.array([-4.0127]))
    assert c.d_rne == 0.0 and c.excess <= 0.0
    c.add_o(np.array([4.0]), np.array([3.998]))
    assert c.excess <= 0.0
