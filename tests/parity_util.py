"""Comparison of device outputs with the float64 oracle, and the parity bars.

Bars (absolute, per element):
  * fp32 outputs: |dO| <= 1e-5 and |dL| <= 1e-5.
  * bf16 outputs: |dL| <= 2e-3 (L is stored in fp32), and for O
        |dO| <= 2e-2                  where |O_ref| < 8,
        |dO| <= spacing_bf16(O_ref)   where |O_ref| >= 8.
    O leaves the kernel rounded to bf16 (nearest even), which alone moves an
    element by up to half the bf16 spacing at its magnitude: 2^-8 |O| at most,
    at most 2^-6 = 0.0156 below |O| = 8, so 2e-2 holds there with room for the
    kernel's own error.  From |O| = 8 on, half a spacing is 2^-5 = 0.031 or
    more, above 2e-2: no bf16 value at all may lie within 2e-2 of O_ref, so
    the bar becomes one spacing there (the output rounding plus as much again
    for the kernel), which matches the room 2e-2 leaves below |O| = 4.
    The workloads keep |O| far below 8; only the wide-score stress inputs
    reach it.

Besides max|dO| each comparison reports two diagnostics that separate the
kernel's error from the output rounding:
  * max |GPU - RNE_bf16(O_ref)|: 0 where the device wrote the correctly
    rounded oracle value;
  * the excess of |GPU - O_ref| over half a bf16 spacing at the stored value,
    a lower bound on the kernel's error before its output rounding.

Bound from the arithmetic (inputs far from the workloads' distribution).
The product W V takes the probabilities rounded to bf16 (relative error at
most 2^-8 each), while O is normalised by the fp32 sum l of the unrounded
weights (which also gives L).  So O moves by at most
delta * sum_j P_ij |V_je| = delta * absmean (the oracle's attention_dev_rows)
through W's rounding.  With delta = 2^-8 + 2^-12 (the rounding, plus fp32
exp2 and score accumulation, each far below 2^-12), fp32 accumulation over n
keys of at most (2 n + 16) 2^-24 (absmean + |O_ie|), and the output rounding
of half a bf16 spacing, every element obeys
    |GPU - O_ref| <= e + spacing(|O_ref| + e) / 2,
    e = delta absmean + (2 n + 16) 2^-24 (absmean + |O_ref|).
The stress tests with peaked rows (keys growing along the sequence; wide
scores with V four times the workloads' scale) assert this bound: there a
dominant weight relative to a base that conditional rescaling left below the
row maximum is not exactly 1, its rounding moves O by up to 2^-8 |O|, and
with |O| near 4 that plus the output rounding passes 2e-2.
"""

import numpy as np

BF16_O, BF16_L = 2e-2, 2e-3
F32_O, F32_L = 1e-5, 1e-5
BF16_WIDE = 8.0  # |O_ref| from which the bar is one bf16 spacing


def bf16_spacing(x):
    """Distance between consecutive bf16 values in the binade of |x| (8
    significant bits): 2^(floor(log2|x|) - 7); 0 where x = 0."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(a)  # a = f 2^e with f in [0.5, 1)
    return np.where(a > 0, np.ldexp(1.0, e - 8), 0.0)


def bf16_rne64(x):
    """float64 values rounded to the nearest bf16 (ties to even), directly
    from float64 (no intermediate fp32 rounding); normal range only."""
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    return np.ldexp(np.rint(f * 256.0) / 256.0, e)


DELTA_W = 2.0 ** -8 + 2.0 ** -12


def rounded_w_bound(o_ref, absmean, n_keys):
    """Per-element bound on |GPU - O_ref| from the arithmetic (module
    docstring); n_keys: keys a row sums over (scalar or per row)."""
    o_ref = np.abs(np.asarray(o_ref, dtype=np.float64))
    n = np.asarray(n_keys, dtype=np.float64)
    if n.ndim == 1:
        n = n[:, None]
    e = DELTA_W * absmean + (2 * n + 16) * 2.0 ** -24 * (absmean + o_ref)
    return e + 0.5 * bf16_spacing(o_ref + e)


def o_bar_bf16(o_ref):
    """Per-element bar on O for bf16 outputs (module docstring)."""
    o_ref = np.asarray(o_ref, dtype=np.float64)
    return np.where(np.abs(o_ref) < BF16_WIDE, BF16_O, np.maximum(BF16_O, bf16_spacing(o_ref)))


class Cmp:
    """Running maxima of the errors of one comparison."""

    def __init__(self, bf16=True):
        self.bf16 = bf16
        self.dO = 0.0         # max |GPU - oracle| over O
        self.o_ratio = 0.0    # max |GPU - oracle| / bar over O
        self.dL = 0.0         # max |GPU - oracle| over L
        self.d_rne = 0.0      # max |GPU - RNE_bf16(oracle)|
        self.excess = 0.0     # max |GPU - oracle| - half spacing at GPU
        self.o_max = 0.0      # max |O_ref|
        self.excess_at = None  # (GPU, oracle) of the element with the largest excess
        self.n = 0

    def add_o(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        d = np.abs(got - ref)
        if d.size == 0:
            return
        self.n += d.size
        self.dO = max(self.dO, float(d.max()))
        self.o_max = max(self.o_max, float(np.abs(ref).max()))
        bar = o_bar_bf16(ref) if self.bf16 else F32_O
        self.o_ratio = max(self.o_ratio, float((d / bar).max()))
        if self.bf16:
            self.d_rne = max(self.d_rne, float(np.abs(got - bf16_rne64(ref)).max()))
            # the largest rounding error that can have produced the stored
            # value: half its binade's spacing (for a power of two, the
            # binade above it, since it may have been rounded down to it)
            g = np.abs(got)
            _, e = np.frexp(g)
            half = np.where(g > 0, np.ldexp(1.0, e - 9), 0.0)
            ex = d - half
            i = int(np.argmax(ex))
            if float(ex.flat[i]) > self.excess:
                self.excess = float(ex.flat[i])
                self.excess_at = (float(got.flat[i]), float(ref.flat[i]))

    def add_l(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        both_inf = np.isneginf(got) & np.isneginf(ref)
        assert np.array_equal(np.isneginf(got), np.isneginf(ref)), "L = -inf must match exactly"
        with np.errstate(invalid="ignore"):
            d = np.abs(np.where(both_inf, 0.0, got - ref))
        if d.size:
            self.dL = max(self.dL, float(d.max()))

    def ok(self):
        return self.o_ratio <= 1.0 and self.dL <= (BF16_L if self.bf16 else F32_L)

    def __repr__(self):
        s = f"max|dO|={self.dO:.3e} (bar ratio {self.o_ratio:.3f}, max|O_ref|={self.o_max:.2f}) max|dL|={self.dL:.3e}"
        if self.bf16:
            s += f" max|GPU-RNE(oracle)|={self.d_rne:.3e} kernel excess>={self.excess:.2e} at {self.excess_at}"
        return s
