"""The polynomial 2^x that the forward can use for part of its exponentials
("Infra: Flash Attention", section "FlashAttention-4": some exponentials on
the multiply-add units, with the approximation error to be evaluated),
checked on the CPU against the mathematics: the instruction sequence that
exact_io_aware_02_amd/gen_fwd_asm.py emits (exp2_poly), evaluated step by
step in float32, against numpy's float64 exp2.

  * relative error at most 8.6e-5 over the fraction's range [0, 1) -- well
    below the 2^-9 of rounding the probabilities to bf16;
  * the error curve equioscillates (four extrema of alternating sign and
    equal size after the fixed p(0) = 1), so the cubic is the best one in
    the maximum-relative-error sense, not merely some cubic that is close;
  * integer exponents are exact (p(0) = 1), masked scores (-inf) and
    anything below -149 give exactly 0, as the hardware exponential does
    at the workloads' scales.
"""

import importlib.util
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def gen():
    spec = importlib.util.spec_from_file_location("_gen_fwd_asm_poly", os.path.join(
        ROOT, "exact_io_aware_02_amd", "gen_fwd_asm.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def _fma32(a, b, c):
    """fp32 fused multiply-add: the float32 product is exact in float64, and
    one rounding of the float64 sum to float32 (the sum's own float64
    rounding is below fp32 resolution for these magnitudes)."""
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(np.float32)


def _poly_exp2(gen, x):
    """The emitted sequence: clamp at POLY_CLAMP, v_fract_f32 (x - floor x,
    at most the largest float below 1), v_cvt_flr_i32_f32, three Horner
    steps (v_fmamk_f32, v_fmaak_f32, v_fma_f32 with 1.0), v_ldexp_f32."""
    c1, c2, c3 = (_f32(getattr(gen, n)) for n in ("POLY_C1", "POLY_C2", "POLY_C3"))
    x = np.maximum(np.asarray(x, np.float32), _f32(gen.POLY_CLAMP))
    fl = np.floor(x)
    f = np.minimum((x - fl).astype(np.float32), np.nextafter(np.float32(1), np.float32(0)))
    p = _fma32(f, c3, c2)
    p = _fma32(p, f, c1)
    p = _fma32(p, f, np.float32(1.0))
    return np.ldexp(p, fl.astype(np.int32)).astype(np.float32)


def _rel_err(gen, x):
    got = _poly_exp2(gen, x).astype(np.float64)
    want = np.exp2(np.asarray(x, np.float64))
    return got / want - 1.0


def test_relative_error_over_the_fraction(gen):
    f = np.linspace(0.0, 1.0, 1 << 20, endpoint=False, dtype=np.float64).astype(np.float32)
    err = np.abs(_rel_err(gen, f))
    assert err.max() <= 8.7e-5, err.max()
    assert err.max() >= 8.0e-5  # a cubic cannot do much better: the fit is not vacuous


def test_error_equioscillates(gen):
    """Local extrema of the relative error of p(f) (float64, so that float32
    rounding does not blur them): after the fixed p(0) = 1, four of them,
    alternating in sign, each within 2 % of the largest."""
    c = [float(_f32(getattr(gen, n))) for n in ("POLY_C1", "POLY_C2", "POLY_C3")]
    f = np.linspace(0.0, 1.0, 200001)
    e = (1.0 + f * (c[0] + f * (c[1] + f * c[2]))) / np.exp2(f) - 1.0
    inner = np.where((np.abs(e[1:-1]) >= np.abs(e[:-2])) & (np.abs(e[1:-1]) >= np.abs(e[2:])))[0] + 1
    ext = [i for i in inner if abs(e[i]) > 0.5 * np.abs(e).max()]
    if abs(e[-1]) > 0.5 * np.abs(e).max():
        ext.append(len(f) - 1)
    vals = e[ext]
    assert len(vals) == 4, vals
    assert np.all(np.sign(vals[1:]) == -np.sign(vals[:-1])), vals
    assert np.abs(vals).min() >= 0.98 * np.abs(vals).max(), vals


def test_whole_range_integers_and_masked_scores(gen):
    # the exponent range of the weights: c (S - m) from far below the base
    # to the conditional-rescale threshold 8 above it
    x = np.linspace(-120.0, 8.0, 400001).astype(np.float32)
    assert np.abs(_rel_err(gen, x)).max() <= 8.7e-5
    k = np.arange(-126, 9).astype(np.float32)
    assert np.array_equal(_poly_exp2(gen, k), np.exp2(k.astype(np.float64)).astype(np.float32))
    dead = np.array([-np.inf, -1e30, -200.0, -150.5, -151.0], dtype=np.float32)
    assert np.array_equal(_poly_exp2(gen, dead), np.zeros(len(dead), np.float32))


def test_every_share_builds_and_uses_the_sequence(gen):
    """Each share replaces exactly that many exponentials per 64 of a tile's
    softmax with the sequence, and the share 0 program has none."""
    for share in (0, *gen.POLY_SHARES):
        sb, wb = gen.S_BUF[0], 0
        pair_tmp = [(gen.TMP0 + 4 * i, gen.TMP0 + 4 * i + 1) for i in range(4)]
        psum = [gen.TMP0 + 4 * (i // 2) + 2 + (i & 1) for i in range(8)]
        ops = gen.exp_ops(sb, wb, pair_tmp, psum, share)
        assert sum(op.startswith("v_ldexp_f32") for op in ops) == share
        assert sum(op.startswith("v_exp_f32") for op in ops) == 64 - share
    with pytest.raises(AssertionError):
        gen.exp_ops(sb, wb, pair_tmp, psum, 5)
