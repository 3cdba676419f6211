"""Parity of the bf16 backward (fa_bwd, through the C ABI) with the float64
oracle (oracle/backward.py).

The forward runs on the GPU first (fa_fwd), as in training: the backward
receives the GPU's O and L.  The oracle gets the same bf16 Q, K, V and dO.

Bar (the pages fix none for the backward; derived from the arithmetic): for
each of dQ, dK, dV and each head, max|GPU - oracle| <= 1e-2 * max|oracle|
+ 1e-5.  The outputs are bf16 (one rounding is up to 2^-9 of the element,
2e-3 of the largest), and P and dS enter the products rounded to bf16;
emulating exactly those roundings on the CPU at these shapes gives 2e-3 to
5e-3 of the largest element, so the relative term leaves a factor of two or
more.  The absolute 1e-5 covers gradients whose exact value cancels to zero
(a single key: dS = P (dP - D) = 0), where fp32 rounding of dP and D leaves
noise of about 1e-7.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

REL, ABS = 1e-2, 1e-5


def _fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_02_amd as fa

    return fa


def _say(*a):
    print("[case]", *a, flush=True)


def _host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _run(Q, K, V, dO, causal, scale=None, workspace=None):
    fa = _fa()
    B, H, N, d = Q.shape
    O = torch.empty_like(Q)
    L = torch.empty(B, H, N, device=Q.device)
    fa.fa_fwd(Q, K, V, O, L, causal=causal, scale=scale)
    dQ, dK, dV = (torch.full_like(Q, float("nan")) for _ in range(3))
    fa.fa_bwd(Q, K, V, O, dO, L, dQ, dK, dV, causal=causal, scale=scale, workspace=workspace)
    torch.cuda.synchronize()
    return O, L, dQ, dK, dV


def _compare(Q, K, V, dO, dQ, dK, dV, causal, scale, heads=None):
    """Worst max|GPU - oracle| / (REL max|oracle| + ABS) over the heads, per
    tensor (the bar is 1)."""
    B, H, N, d = Q.shape
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    worst = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
    for b, h in heads:
        ref = oracle.attention_backward(_host(Q[b, h]), _host(K[b, h]), _host(V[b, h]), _host(dO[b, h]), scale,
                                        causal=causal)
        for name, got, r in (("dQ", dQ, ref[0]), ("dK", dK, ref[1]), ("dV", dV, ref[2])):
            g = _host(got[b, h])
            assert np.all(np.isfinite(g)), (name, b, h)
            worst[name] = max(worst[name], float(np.max(np.abs(g - r)) / (REL * np.max(np.abs(r)) + ABS)))
    return worst


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 65, 127, 128, 129, 300])
def test_bwd_small_shapes(N, d, causal):
    _say("bwd", N, d, causal)
    shape = (2, 2, N, d)
    Q, K, V, dO = (synth.torch_normal(800 + t, shape, "cuda", "bf16") for t in range(4))
    _, _, dQ, dK, dV = _run(Q, K, V, dO, causal)
    worst = _compare(Q, K, V, dO, dQ, dK, dV, causal, 1 / math.sqrt(d))
    print(f"N={N} d={d} causal={causal} {worst}")
    assert max(worst.values()) <= 1.0, worst


def test_bwd_wide_scores_and_scale():
    """Values x4 and scale 0.05: peaked rows, where P is close to one-hot."""
    _say("bwd wide scores")
    shape = (1, 2, 333, 128)
    Q, K, V, dO = (synth.torch_normal(820 + t, shape, "cuda", "bf16", vscale=4.0) for t in range(4))
    for causal in (False, True):
        _, _, dQ, dK, dV = _run(Q, K, V, dO, causal, scale=0.05)
        worst = _compare(Q, K, V, dO, dQ, dK, dV, causal, 0.05)
        assert max(worst.values()) <= 1.0, (causal, worst)


def test_bwd_workspace_and_determinism():
    """The caller's workspace and the internal one give identical bits, and
    two runs give identical bits (no atomics)."""
    fa = _fa()
    _say("bwd workspace / determinism")
    shape = (2, 3, 500, 128)
    Q, K, V, dO = (synth.torch_normal(830 + t, shape, "cuda", "bf16") for t in range(4))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(2, 3, 500), dtype=torch.uint8, device="cuda")
    for causal in (False, True):
        a = _run(Q, K, V, dO, causal)
        b = _run(Q, K, V, dO, causal, workspace=ws)
        for x, y in zip(a[2:], b[2:]):
            assert torch.equal(x, y), causal


def test_bwd_single_key_closed_form():
    """N = 1: P = [[1]], so dV = dO (rounded to bf16, already bf16) and
    dQ = dK = 0 up to fp32 noise in dP - D."""
    _say("bwd N=1 closed form")
    shape = (1, 4, 1, 128)
    Q, K, V, dO = (synth.torch_normal(840 + t, shape, "cuda", "bf16") for t in range(4))
    _, _, dQ, dK, dV = _run(Q, K, V, dO, False)
    assert torch.equal(dV, dO)
    assert dQ.float().abs().max().item() <= ABS and dK.float().abs().max().item() <= ABS


@pytest.mark.parametrize("name", ["prefill_8k", "causal_4k"])
def test_bwd_workload_shapes(name):
    """The prefill workloads' shapes, as the bench times them, compared on
    two whole heads (first and last)."""
    cfg = synth.WORKLOADS[name]
    _say("bwd workload", name, cfg)
    Q, K, V = synth.prefill_inputs(name, "cuda")
    dO = synth.torch_normal(850, tuple(Q.shape), "cuda", "bf16")
    causal = cfg["causal"]
    _, _, dQ, dK, dV = _run(Q, K, V, dO, causal)
    B, H = cfg["B"], cfg["H"]
    worst = _compare(Q, K, V, dO, dQ, dK, dV, causal, 1 / math.sqrt(cfg["d"]), heads=[(0, 0), (B - 1, H - 1)])
    print(f"{name} {worst}")
    assert max(worst.values()) <= 1.0, worst


def test_bwd_long_sequence_one_head():
    """N = 16384 non-causal and causal, one head compared in full."""
    _say("bwd N=16384")
    shape = (1, 1, 16384, 128)
    Q, K, V, dO = (synth.torch_normal(860 + t, shape, "cuda", "bf16") for t in range(4))
    for causal in (False, True):
        _, _, dQ, dK, dV = _run(Q, K, V, dO, causal)
        worst = _compare(Q, K, V, dO, dQ, dK, dV, causal, 1 / math.sqrt(128))
        print(f"N=16384 causal={causal} {worst}")
        assert max(worst.values()) <= 1.0, (causal, worst)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [100, 1000])
def test_bwd_ragged_tail_reads_nothing_past_the_head(N, causal):
    """Rows past N are not part of the problem: the backward's Q, dO, K, V
    tiles and its L and D rows must read them as zeros, never as whatever
    memory follows the last head.  Every input is a view at the start of an
    allocation whose remainder holds NaN, so a read past the last head would
    turn into NaN in a gradient; the reads stay inside the allocation either
    way."""
    fa = _fa()
    _say("bwd ragged tail guard", N, causal)
    shape = (1, 3, N, 128)
    n = math.prod(shape)
    views = []
    for t in range(4):
        buf = torch.full((n + 256 * 128,), float("nan"), device="cuda", dtype=torch.bfloat16)
        buf[:n] = synth.torch_normal(830 + t, shape, "cuda", "bf16").reshape(-1)
        views.append(buf[:n].view(shape))
    Q, K, V, dO = views
    obuf = torch.full((n + 256 * 128,), float("nan"), device="cuda", dtype=torch.bfloat16)
    lbuf = torch.full((3 * N + 256,), float("nan"), device="cuda")
    O, L = obuf[:n].view(shape), lbuf[:3 * N].view(shape[:3])
    fa.fa_fwd(Q, K, V, O, L, causal=causal)
    dQ, dK, dV = (torch.full_like(Q, float("nan")) for _ in range(3))
    fa.fa_bwd(Q, K, V, O, dO, L, dQ, dK, dV, causal=causal)
    torch.cuda.synchronize()
    worst = _compare(Q, K, V, dO, dQ, dK, dV, causal, 1 / math.sqrt(128))
    assert max(worst.values()) <= 1.0, worst
