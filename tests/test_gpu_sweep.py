"""A seeded sweep of random problem shapes through the C ABI, against the
float64 oracle, beside the hand-picked shapes of the other GPU tests: head
counts, lengths (1 to about 1,500, so single-tile, ragged and multi-item
launches), head dimension 64 or 128, causal or not, the scale passed in or
the default 1/sqrt(d), value scales, and for decode the split count, empty
caches and the padded layout.  Every element of every output is compared.

The configurations are drawn once from a fixed seed, so a failure names a
case that reproduces.  Score spreads stay within about three times the
workloads' (scale * sqrt(d) * vscale^2 <= 2.3), where the flat bf16 bars
apply; the peaked-row stress inputs are tested against the bound from the
arithmetic in test_gpu_parity.py."""

import math

import numpy as np
import pytest
import torch

import synth
from tests.test_gpu_backward import REL, _compare as _bwd_compare, _run as _bwd_run
from tests.test_gpu_parity import _decode_compare, _prefill_compare

pytestmark = pytest.mark.gpu


def _fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_02_amd as fa

    return fa


def _say(*a):
    print("[case]", *a, flush=True)


def _length(rng, i, hi):
    """Lengths over the scales that matter, by stratum i % 3: below one
    tile, a few tiles, many tiles (log-uniform in [1, 64), [64, hi / 3),
    [hi / 3, hi])."""
    lo, up = ((1, 64), (64, hi // 3), (hi // 3, hi))[i % 3]
    return int(np.exp(rng.uniform(math.log(lo), math.log(up))))


def _prefill_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        vscale = float(rng.choice([0.5, 1.0]))
        scale = None if rng.random() < 0.4 else float(rng.uniform(0.03, 0.2))
        out.append(dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 5)), N=_length(rng, i, 1500), d=d,
                        causal=bool(rng.random() < 0.5), scale=scale, vscale=vscale, seed=9000 + 10 * i))
    return out


def _decode_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 5))
        lengths = [0 if rng.random() < 0.15 else _length(rng, i + k, 3000) for k in range(B)]
        out.append(dict(B=B, H=int(rng.integers(1, 7)), d=int(rng.choice([64, 128])), lengths=lengths,
                        splits=int(rng.choice([0, 1, int(rng.integers(2, 41))])),
                        padded=bool(rng.random() < 0.4), scale=None if rng.random() < 0.5 else
                        float(rng.uniform(0.03, 0.2)), seed=9500 + 10 * i))
    return out


def _backward_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        out.append(dict(H=int(rng.integers(1, 4)), N=_length(rng, i, 500), d=int(rng.choice([64, 128])),
                        causal=bool(rng.random() < 0.5),
                        scale=None if rng.random() < 0.5 else float(rng.uniform(0.03, 0.2)), seed=9800 + 10 * i))
    return out


PREFILL = _prefill_cases(16, 2026)
FP32 = [dict(c, vscale=1.0, d=(64, 128)[i % 2]) for i, c in enumerate(_prefill_cases(6, 2027))]
DECODE = _decode_cases(10, 2028)
BACKWARD = _backward_cases(6, 2029)


def _ids(cases, keys):
    return ["-".join(f"{k}{c[k]}" for k in keys) for c in cases]


@pytest.mark.parametrize("case", PREFILL, ids=_ids(PREFILL, ("B", "H", "N", "d", "causal")))
def test_sweep_prefill_bf16(case):
    fa = _fa()
    _say("sweep prefill bf16", case)
    shape = (case["B"], case["H"], case["N"], case["d"])
    Q, K, V = (synth.torch_normal(case["seed"] + t, shape, "cuda", "bf16", vscale=case["vscale"]) for t in range(3))
    O = torch.full_like(Q, float("nan"))
    L = torch.full(shape[:3], float("nan"), device="cuda")
    fa.fa_fwd(Q, K, V, O, L, causal=case["causal"], scale=case["scale"])
    torch.cuda.synchronize()
    scale = case["scale"] or 1 / math.sqrt(case["d"])
    c = _prefill_compare(Q, K, V, O, L, scale, case["causal"])
    assert c.ok(), c


@pytest.mark.parametrize("case", FP32, ids=_ids(FP32, ("B", "H", "N", "d", "causal")))
def test_sweep_prefill_fp32(case):
    fa = _fa()
    _say("sweep prefill fp32", case)
    shape = (case["B"], case["H"], case["N"], case["d"])
    Q, K, V = (synth.torch_normal(case["seed"] + t, shape, "cuda", "f32") for t in range(3))
    O = torch.full_like(Q, float("nan"))
    L = torch.full(shape[:3], float("nan"), device="cuda")
    fa.fa_fwd_f32(Q, K, V, O, L, causal=case["causal"], scale=case["scale"])
    torch.cuda.synchronize()
    scale = case["scale"] or 1 / math.sqrt(case["d"])
    c = _prefill_compare(Q, K, V, O, L, scale, case["causal"])
    assert c.ok(), c


@pytest.mark.parametrize("case", DECODE, ids=_ids(DECODE, ("B", "H", "d", "splits", "padded")))
def test_sweep_decode(case):
    fa = _fa()
    _say("sweep decode", case)
    B, H, d = case["B"], case["H"], case["d"]
    lengths = np.array(case["lengths"], dtype=np.int64)
    q = synth.torch_normal(case["seed"], (B, H, d), "cuda")
    if case["padded"]:
        cap = int(lengths.max()) + 37
        Kc = synth.torch_normal(case["seed"] + 1, (B, H, cap, d), "cuda")
        Vc = synth.torch_normal(case["seed"] + 2, (B, H, cap, d), "cuda")
    else:
        cap = 0
        total = max(int(lengths.sum()), 1) * H * d
        Kc = synth.torch_normal(case["seed"] + 1, (total,), "cuda")
        Vc = synth.torch_normal(case["seed"] + 2, (total,), "cuda")
    Lkv = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H), float("nan"), device="cuda")
    ws = torch.empty(fa.fa_decode_workspace_bytes(B, H, d, case["splits"]), dtype=torch.uint8, device="cuda")
    fa.fa_decode_ex(q, Kc, Vc, o, Lkv, ws, lse_out=lse, kv_seq_capacity=cap, num_splits=case["splits"],
                    scale=case["scale"])
    torch.cuda.synchronize()
    c = _decode_compare(q, Kc, Vc, o, lengths, lse=lse, scale=case["scale"], capacity=cap)
    assert c.ok(), c
    for b in np.flatnonzero(lengths == 0):   # an empty cache: o = 0, lse = -inf
        assert torch.all(o[b] == 0) and torch.all(torch.isneginf(lse[b]))


@pytest.mark.parametrize("case", BACKWARD, ids=_ids(BACKWARD, ("H", "N", "d", "causal")))
def test_sweep_backward(case):
    _fa()
    _say("sweep backward", case)
    shape = (1, case["H"], case["N"], case["d"])
    Q, K, V, dO = (synth.torch_normal(case["seed"] + t, shape, "cuda", "bf16") for t in range(4))
    _, _, dQ, dK, dV = _bwd_run(Q, K, V, dO, case["causal"], scale=case["scale"])
    scale = case["scale"] or 1 / math.sqrt(case["d"])
    worst = _bwd_compare(Q, K, V, dO, dQ, dK, dV, case["causal"], scale)
    assert max(worst.values()) <= 1.0, (worst, REL)


def test_sweep_cases_cover_the_edges():
    """The draw includes the shapes the sweep is for (checked on the host)."""
    assert any(c["N"] < 64 for c in PREFILL) and any(c["N"] > 700 for c in PREFILL)
    assert any(c["causal"] for c in PREFILL) and any(not c["causal"] for c in PREFILL)
    assert {c["d"] for c in PREFILL} == {64, 128} and any(c["scale"] is None for c in PREFILL)
    assert {c["d"] for c in FP32} == {64, 128} and any(c["N"] > 500 for c in FP32)
    assert any(0 in c["lengths"] for c in DECODE) and any(c["padded"] for c in DECODE)
    assert {c["splits"] for c in DECODE} & {0, 1} and any(c["splits"] > 1 for c in DECODE)
    assert any(c["causal"] for c in BACKWARD) and any(not c["causal"] for c in BACKWARD)
