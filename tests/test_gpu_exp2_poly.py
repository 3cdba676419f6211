"""Parity of the d = 128 bf16 forward when part of its exponentials run as a
polynomial on the multiply-add units ("Infra: Flash Attention", section
"FlashAttention-4"; fa_set_fwd_exp2_poly), through the C ABI, against the
float64 oracle with the same bars as the hardware-exponential kernel
(tests/parity_util.py).  The polynomial's relative error (8.6e-5, pinned on
the CPU by tests/test_exp2_poly.py) is below the bf16 rounding of the
probabilities, which the bars already allow for."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

from tests.parity_util import BF16_L, Cmp, rounded_w_bound

SHARES = (4, 8, 16)


def _fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_02_amd as fa

    return fa


def _say(*a):
    print("[case]", *a, flush=True)


def _host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


class _share:
    """Runs the forward with `per64` exponentials per 64 by polynomial and
    restores the previous setting."""

    def __init__(self, fa, per64):
        self.fa, self.per64 = fa, per64

    def __enter__(self):
        self.prev = self.fa.fa_set_fwd_exp2_poly(self.per64)
        assert self.fa.fa_get_fwd_exp2_poly() == self.per64

    def __exit__(self, *exc):
        self.fa.fa_set_fwd_exp2_poly(self.prev)


def _compare(Q, K, V, O, L, scale, causal):
    B, H, N, _ = Q.shape
    c = Cmp(bf16=True)
    for b in range(B):
        for h in range(H):
            o_ref, l_ref = oracle.attention_rows(_host(Q[b, h]), _host(K[b, h]), _host(V[b, h]), scale,
                                                 causal=causal)
            c.add_o(_host(O[b, h]), o_ref)
            c.add_l(_host(L[b, h]), l_ref)
    return c


def _run(fa, per64, Q, K, V, causal, scale=None):
    O = torch.full_like(Q, float("nan"))
    L = torch.full(Q.shape[:3], float("nan"), device="cuda")
    with _share(fa, per64):
        fa.fa_fwd(Q, K, V, O, L, causal=causal, scale=scale)
        torch.cuda.synchronize()
    return O, L


@pytest.mark.parametrize("per64", SHARES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 64, 129, 1000])
def test_poly_small_shapes(N, causal, per64):
    """Several tiles, a ragged last tile, a single key; every element."""
    fa = _fa()
    _say("exp2 poly", per64, N, causal)
    shape = (2, 2, N, 128)
    Q, K, V = (synth.torch_normal(200 + t, shape, "cuda", "bf16") for t in range(3))
    O, L = _run(fa, per64, Q, K, V, causal)
    c = _compare(Q, K, V, O, L, 1 / math.sqrt(128), causal)
    assert c.ok(), c


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N", [(1, 300, 300), (1, 3, 2113)])
def test_poly_many_items(B, H, N, causal):
    """Persistent workgroups running sequences of items, long rows with a
    ragged tail (causal: skipped products after a wavefront's rows);
    every element."""
    fa = _fa()
    _say("exp2 poly many items", B, H, N, causal)
    shape = (B, H, N, 128)
    Q, K, V = (synth.torch_normal(700 + t, shape, "cuda", "bf16") for t in range(3))
    O, L = _run(fa, 16, Q, K, V, causal)
    assert not torch.isnan(O).any() and not torch.isnan(L).any()
    c = _compare(Q, K, V, O, L, 1 / math.sqrt(128), causal)
    assert c.ok(), c


@pytest.mark.parametrize("per64", SHARES)
def test_poly_base_moves_and_wide_scores(per64):
    """Peaked rows whose base moves in later tiles (keys growing along the
    sequence), and widely spread scores: held to the bound from the
    kernel's arithmetic (rounded_w_bound), whose 2^-12 allowance for the
    exponential covers the polynomial's 8.6e-5."""
    fa = _fa()
    _say("exp2 poly base moves / wide scores", per64)
    N = 1000
    shape = (1, 2, N, 128)
    Q, K, V = (synth.torch_normal(800 + t, shape, "cuda", "f32") for t in range(3))
    ramp = 1.0 + 7.0 * torch.arange(N, device="cuda", dtype=torch.float32) / N
    K = K * ramp[None, None, :, None]
    ramped = tuple(t.to(torch.bfloat16) for t in (Q, K, V))
    wide = tuple(synth.torch_normal(300 + t, (1, 2, 777, 128), "cuda", "bf16", vscale=4.0) for t in range(3))
    for name, (Qx, Kx, Vx), scale in (("base moves", ramped, 1 / math.sqrt(128)), ("wide", wide, 0.05)):
        n = Qx.shape[2]
        for causal in (False, True):
            O, L = _run(fa, per64, Qx, Kx, Vx, causal, scale)
            worst = 0.0
            c = Cmp(bf16=True)
            n_keys = np.arange(1, n + 1) if causal else np.full(n, n)
            for h in range(Qx.shape[1]):
                q, k, v = _host(Qx[0, h]), _host(Kx[0, h]), _host(Vx[0, h])
                o_ref, l_ref = oracle.attention_rows(q, k, v, scale, causal=causal)
                _, am = oracle.attention_dev_rows(q, k, v, scale, causal=causal)
                got = _host(O[0, h])
                c.add_o(got, o_ref)
                c.add_l(_host(L[0, h]), l_ref)
                worst = max(worst, float(np.max(np.abs(got - o_ref) / rounded_w_bound(o_ref, am, n_keys))))
            print(name, "causal" if causal else "", c, f"| worst |dO|/bound = {worst:.3f}")
            assert worst <= 1.0 and c.dL <= BF16_L, (name, causal, worst, c)


@pytest.mark.parametrize("workload,causal", [("prefill_8k", False), ("causal_4k", True)])
def test_poly_workloads_all_elements(workload, causal):
    """The two prefill workloads with the largest share, every element
    against the oracle; beside it, how far the outputs move from the
    hardware-exponential kernel's (printed)."""
    fa = _fa()
    cfg = synth.WORKLOADS[workload]
    _say("exp2 poly workload", workload)
    Q, K, V = synth.prefill_inputs(workload, "cuda")
    O, L = _run(fa, 16, Q, K, V, causal)
    O0, L0 = _run(fa, 0, Q, K, V, causal)
    assert torch.isfinite(O).all() and torch.isfinite(L).all()
    if causal:
        assert torch.equal(O[:, :, 0], V[:, :, 0])
    print(workload, "max |O_poly - O_exp| =", float((O.float() - O0.float()).abs().max()),
          "max |L_poly - L_exp| =", float((L - L0).abs().max()), flush=True)
    c = _compare(Q, K, V, O, L, 1 / math.sqrt(cfg["d"]), causal)
    print(workload, c, flush=True)
    assert c.n == Q.numel()
    assert c.ok(), c


def test_poly_setting_is_validated_and_default_is_off():
    fa = _fa()
    assert fa.fa_get_fwd_exp2_poly() == 0
    with pytest.raises(fa.FAError):
        fa.fa_set_fwd_exp2_poly(3)
    assert fa.fa_get_fwd_exp2_poly() == 0
