"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Bars (tests/parity_util.py): bf16 inputs -- |dO| <= 2e-2 (one bf16 spacing
where |O| >= 8, since the bf16 output alone may then be more than 2e-2 away)
and |dL| <= 2e-3; fp32 inputs -- |dO| <= 1e-5 and |dL| <= 1e-5 (absolute,
per element).  Small shapes and the five workloads are compared element by
element, the workloads in the launch configuration the bench times; only the
inputs larger than the workloads are compared on sampled rows.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

from tests.parity_util import BF16_L, BF16_O, Cmp, rounded_w_bound


def _fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_02_amd as fa

    return fa


def _say(*a):
    print("[case]", *a, flush=True)


def _host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _prefill_compare(Q, K, V, O, L, scale, causal, rows=None, heads=None):
    """Compare device outputs with the oracle on the given (b, h) heads and
    query rows (all when None).  Returns a Cmp (bf16 bars unless Q is fp32)."""
    B, H, N, d = Q.shape
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    c = Cmp(bf16=Q.dtype != torch.float32)
    r = np.arange(N) if rows is None else np.asarray(rows)
    ri = None if rows is None else torch.as_tensor(r, device=Q.device)
    for b, h in heads:
        pick = (lambda t: t[b, h]) if ri is None else (lambda t: t[b, h, ri])
        k, v = _host(K[b, h]), _host(V[b, h])
        o_ref, l_ref = oracle.attention_rows(_host(pick(Q)), k, v, scale, causal=causal, q_pos=r)
        c.add_o(_host(pick(O)), o_ref)
        c.add_l(_host(pick(L)), l_ref)
    return c


# --------------------------------------------------------------------------
# fp32 path
# --------------------------------------------------------------------------

def test_fp32_small_workload_all_elements():
    fa = _fa()
    cfg = synth.WORKLOADS["fp32_small"]
    _say("fp32_small", cfg)
    Q, K, V = synth.prefill_inputs("fp32_small", "cuda")
    O = torch.empty_like(Q)
    L = torch.empty(Q.shape[:3], device="cuda", dtype=torch.float32)
    scale = 1.0 / math.sqrt(cfg["d"])
    fa.fa_fwd_f32(Q, K, V, O, L, causal=False, scale=scale)
    torch.cuda.synchronize()
    c = _prefill_compare(Q, K, V, O, L, scale, False)
    print("fp32_small", c)
    assert c.ok(), c


def test_fp32_worked_example_49_over_15():
    """'Infra: Flash Attention', worked example of the state merge: scores
    log 1, log 2, log 4, log 8 against values 1, 2, 3, 4 give 49/15 and
    L = log 15."""
    fa = _fa()
    _say("fp32 49/15 example")
    d, N = 64, 4
    Q = torch.zeros(1, 1, N, d, device="cuda")
    K = torch.zeros_like(Q)
    V = torch.zeros_like(Q)
    Q[0, 0, :, 0] = 1.0
    K[0, 0, :, 0] = torch.tensor([math.log(1), math.log(2), math.log(4), math.log(8)])
    V[0, 0, :, 0] = torch.tensor([1.0, 2.0, 3.0, 4.0])
    O = torch.empty_like(Q)
    L = torch.empty(1, 1, N, device="cuda")
    fa.fa_fwd_f32(Q, K, V, O, L, causal=False, scale=1.0)
    torch.cuda.synchronize()
    assert abs(O[0, 0, 0, 0].item() - 49 / 15) <= 1e-6
    assert abs(L[0, 0, 0].item() - math.log(15)) <= 1e-6


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 63, 65, 200, 700])
def test_fp32_small_shapes(N, d, causal):
    fa = _fa()
    _say("fp32", N, d, causal)
    shape = (2, 3, N, d)
    Q, K, V = (synth.torch_normal(100 + t, shape, "cuda", "f32") for t in range(3))
    O = torch.empty_like(Q)
    L = torch.empty(shape[:3], device="cuda")
    fa.fa_fwd_f32(Q, K, V, O, L, causal=causal)
    torch.cuda.synchronize()
    c = _prefill_compare(Q, K, V, O, L, 1 / math.sqrt(d), causal)
    assert c.ok(), c


# --------------------------------------------------------------------------
# bf16 prefill
# --------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 127, 128, 129, 300, 1000])
def test_bf16_small_shapes(N, d, causal):
    fa = _fa()
    _say("bf16", N, d, causal)
    shape = (2, 2, N, d)
    Q, K, V = (synth.torch_normal(200 + t, shape, "cuda", "bf16") for t in range(3))
    O = torch.empty_like(Q)
    L = torch.empty(shape[:3], device="cuda")
    fa.fa_fwd(Q, K, V, O, L, causal=causal)
    torch.cuda.synchronize()
    c = _prefill_compare(Q, K, V, O, L, 1 / math.sqrt(d), causal)
    assert c.ok(), c


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [17, 100, 1000])
def test_bf16_ragged_tail_reads_nothing_past_the_head(N, d):
    """Keys past N are not part of the problem: their rows must read as
    zeros, never as whatever memory follows the head.  Q, K, V are views at
    the start of one allocation whose remainder holds NaN, so any read past
    the last head would turn into NaN in O (a NaN value row times a zero
    weight is still NaN); the reads stay inside the allocation either way."""
    fa = _fa()
    _say("bf16 ragged tail guard", N, d)
    shape = (1, 3, N, d)
    n = math.prod(shape)
    outs = []
    for t in range(3):
        buf = torch.full((n + 128 * d,), float("nan"), device="cuda", dtype=torch.bfloat16)
        buf[:n] = synth.torch_normal(500 + t, shape, "cuda", "bf16").reshape(-1)
        outs.append(buf[:n].view(shape))
    Q, K, V = outs
    O = torch.empty_like(Q)
    L = torch.empty(shape[:3], device="cuda")
    for causal in (False, True):
        fa.fa_fwd(Q, K, V, O, L, causal=causal)
        torch.cuda.synchronize()
        assert not torch.isnan(O).any() and not torch.isnan(L).any(), causal
        c = _prefill_compare(Q, K, V, O, L, 1 / math.sqrt(d), causal)
        assert c.ok(), (causal, c)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,H,N", [(2, 200, 50), (1, 300, 300), (1, 520, 129), (3, 100, 700),
                                   (1, 257, 513), (1, 3, 2113)])
def test_bf16_many_items_per_workgroup(B, H, N, causal):
    """At d = 128 launches keep at most one workgroup per compute unit, so
    with many heads each workgroup runs a sequence of query tiles (causal:
    pairs of them) whose heads change from one to the next.  An item's last
    product block loads the next item's Q, K_0 and K_1, and the next item
    waits for them behind the previous item's stores.  Causal: a wavefront
    skips the products of tiles after its rows, whole steps two tiles past
    its diagonal one, and the final block when the last tile is after its
    rows.  Covers single-tile items (N <= 64: every step is an item
    boundary), ragged last tiles, a grid with fewer items than compute units
    in its last round (257 x 3 tiles over 256 workgroups), long items with
    a ragged tail (N = 2113: 9 query tiles, up to 34 steps) and mixes of long
    and short items; every head and row is compared."""
    fa = _fa()
    _say("bf16 many items", B, H, N, "causal" if causal else "non-causal")
    shape = (B, H, N, 128)
    Q, K, V = (synth.torch_normal(700 + t, shape, "cuda", "bf16") for t in range(3))
    O = torch.full_like(Q, float("nan"))
    L = torch.full(shape[:3], float("nan"), device="cuda")
    fa.fa_fwd(Q, K, V, O, L, causal=causal)
    torch.cuda.synchronize()
    assert not torch.isnan(O).any() and not torch.isnan(L).any()
    c = _prefill_compare(Q, K, V, O, L, 1 / math.sqrt(128), causal)
    assert c.ok(), c


def _bound_compare(Q, K, V, O, L, scale, causal):
    """(max over elements of |GPU - oracle| / the bound from the arithmetic,
    the flat-bar comparison) for every head and row."""
    B, H, N, d = Q.shape
    c = _prefill_compare(Q, K, V, O, L, scale, causal)
    worst = 0.0
    n_keys = np.arange(1, N + 1) if causal else np.full(N, N)
    for b in range(B):
        for h in range(H):
            q, k, v = _host(Q[b, h]), _host(K[b, h]), _host(V[b, h])
            o_ref, _ = oracle.attention_rows(q, k, v, scale, causal=causal)
            _, am = oracle.attention_dev_rows(q, k, v, scale, causal=causal)
            bound = rounded_w_bound(o_ref, am, n_keys)
            worst = max(worst, float(np.max(np.abs(_host(O[b, h]) - o_ref) / bound)))
    return worst, c


def test_bf16_large_values_and_scale():
    """Scores with a wide spread (values x4, scale 0.05: score std about 9)
    exercise the running maximum and the alpha rescale across many tiles.
    These inputs are far from the workloads' N(0,1): rows are peaked and |O|
    reaches about 16, so rounding the probabilities to bf16 for the W V
    product alone can move O by more than 2e-2.  Every element is held to the
    bound that follows from the kernel's arithmetic (tests/parity_util.py,
    rounded_w_bound); the flat-bar comparison is printed beside it."""
    fa = _fa()
    _say("bf16 wide scores")
    shape = (1, 2, 777, 128)
    N = shape[2]
    Q, K, V = (synth.torch_normal(300 + t, shape, "cuda", "bf16", vscale=4.0) for t in range(3))
    O = torch.empty_like(Q)
    L = torch.empty(shape[:3], device="cuda")
    for causal in (False, True):
        fa.fa_fwd(Q, K, V, O, L, causal=causal, scale=0.05)
        torch.cuda.synchronize()
        worst, c = _bound_compare(Q, K, V, O, L, 0.05, causal)
        print("wide scores causal" if causal else "wide scores", c, f"| worst |dO|/bound = {worst:.3f}")
        assert worst <= 1.0 and c.dL <= BF16_L, (causal, worst, c)


@pytest.mark.parametrize("N", [1000, 2049])
def test_bf16_base_moves_in_later_tiles(N):
    """Keys grow along the sequence (key j scaled by 1 + 7 j / N), so later
    KV tiles hold scores far above the first tile's maximum: the running base
    moves mid-row, after U and l have been accumulated, and U and l must be
    rescaled ("Invariant of conditional rescaling").  The rows are peaked, O
    is nearly one row of V (|O| up to about 4.2), and a dominant weight
    relative to a base left below the row maximum is not exactly 1: its bf16
    rounding moves O by up to 2^-8 |O| on top of the output rounding (up to
    0.0156 at |O| >= 4).  Every element is held to the bound that follows
    from the kernel's arithmetic (tests/parity_util.py, rounded_w_bound), L
    to 2e-3; the flat-bar comparison is printed beside it."""
    fa = _fa()
    _say("bf16 base moves in later tiles", N)
    shape = (1, 4, N, 128)
    Q, K, V = (synth.torch_normal(800 + t, shape, "cuda", "f32") for t in range(3))
    ramp = 1.0 + 7.0 * torch.arange(N, device="cuda", dtype=torch.float32) / N
    K = K * ramp[None, None, :, None]
    Q, K, V = (t.to(torch.bfloat16) for t in (Q, K, V))
    O = torch.empty_like(Q)
    L = torch.empty(shape[:3], device="cuda")
    for causal in (False, True):
        fa.fa_fwd(Q, K, V, O, L, causal=causal)
        torch.cuda.synchronize()
        worst, c = _bound_compare(Q, K, V, O, L, 1 / math.sqrt(128), causal)
        print("base moves", N, "causal" if causal else "", c, f"| worst |dO|/bound = {worst:.3f}")
        assert worst <= 1.0 and c.dL <= BF16_L, (causal, worst, c)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_L_optional_and_deterministic(causal, d):
    """O does not depend on whether L is requested (L = NULL: the kernels'
    L stores go nowhere), and repeated launches give the same bits."""
    fa = _fa()
    _say("bf16 determinism", causal, d)
    shape = (1, 4, 1000, d)
    Q, K, V = (synth.torch_normal(400 + t, shape, "cuda", "bf16") for t in range(3))
    O1, O2, O3 = torch.empty_like(Q), torch.empty_like(Q), torch.empty_like(Q)
    L1, L3 = torch.empty(shape[:3], device="cuda"), torch.empty(shape[:3], device="cuda")
    fa.fa_fwd(Q, K, V, O1, L1, causal=causal)
    fa.fa_fwd(Q, K, V, O2, None, causal=causal)
    fa.fa_fwd(Q, K, V, O3, L3, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(O1, O3) and torch.equal(L1, L3)


def _rows_sample(N, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, N // 2, N - 129, N - 128, N - 65, N - 64, N - 2, N - 1]
    return np.unique(np.concatenate([fixed, rng.integers(0, N, 32)]))


def test_bf16_prefill_8k_workload_all_elements():
    """The prefill_8k workload in the bench's launch configuration, every
    head and row against the oracle."""
    fa = _fa()
    cfg = synth.WORKLOADS["prefill_8k"]
    _say("prefill_8k", cfg)
    Q, K, V = synth.prefill_inputs("prefill_8k", "cuda")
    O = torch.empty_like(Q)
    L = torch.empty(Q.shape[:3], device="cuda")
    fa.fa_fwd(Q, K, V, O, L, causal=False)
    torch.cuda.synchronize()
    assert torch.isfinite(O).all() and torch.isfinite(L).all()
    c = _prefill_compare(Q, K, V, O, L, 1 / math.sqrt(cfg["d"]), False)
    print("prefill_8k", c, flush=True)
    assert c.n == Q.numel()
    assert c.ok(), c


def test_bf16_causal_4k_workload_all_elements():
    """The causal_4k workload in the bench's launch configuration, every
    (b, h) and row against the oracle."""
    fa = _fa()
    cfg = synth.WORKLOADS["causal_4k"]
    _say("causal_4k", cfg)
    Q, K, V = synth.prefill_inputs("causal_4k", "cuda")
    O = torch.empty_like(Q)
    L = torch.empty(Q.shape[:3], device="cuda")
    fa.fa_fwd(Q, K, V, O, L, causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(O).all() and torch.isfinite(L).all()
    # causal row 0 sees only key 0: O_0 = V_0 exactly up to output rounding
    assert torch.equal(O[:, :, 0], V[:, :, 0])
    c = _prefill_compare(Q, K, V, O, L, 1 / math.sqrt(cfg["d"]), True)
    print("causal_4k", c, flush=True)
    assert c.n == Q.numel()
    assert c.ok(), c


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------

def _decode_oracle(q, Kc, Vc, lengths, H, d, b, h, scale, capacity=0):
    if capacity:
        base = (b * H + h) * capacity * d
    else:
        base = int(synth.packed_offsets(lengths, H, d)[b]) + h * int(lengths[b]) * d
    Lb = int(lengths[b])
    k = _host(Kc.view(-1)[base:base + Lb * d]).reshape(Lb, d)
    v = _host(Vc.view(-1)[base:base + Lb * d]).reshape(Lb, d)
    return oracle.decode_ref(_host(q[b, h]), k, v, scale)


def _decode_compare(q, Kc, Vc, o, lengths, lse=None, pairs=None, scale=None, capacity=0):
    """Compare o (and lse when given) with the oracle on the given (b, h)
    pairs (all when None).  Returns a Cmp."""
    B, H, d = q.shape
    scale = scale or 1 / math.sqrt(d)
    pairs = pairs if pairs is not None else [(b, h) for b in range(B) for h in range(H)]
    c = Cmp(bf16=True)
    for b, h in pairs:
        o_ref, l_ref = _decode_oracle(q, Kc, Vc, lengths, H, d, b, h, scale, capacity)
        c.add_o(_host(o[b, h]), o_ref)
        if lse is not None:
            c.add_l(np.array([float(lse[b, h].item())]), np.array([l_ref]))
    return c


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("splits", [1, 3, 7, 64, 0])
def test_decode_small(d, splits):
    fa = _fa()
    _say("decode small", d, splits)
    lengths = np.array([1, 63, 1000, 0, 200], dtype=np.int64)
    B, H = len(lengths), 3
    total = int(lengths.sum()) * H * d
    q = synth.torch_normal(500, (B, H, d), "cuda")
    Kc = synth.torch_normal(501, (total,), "cuda")
    Vc = synth.torch_normal(502, (total,), "cuda")
    Lkv = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    fa.fa_decode(q, Kc, Vc, o, Lkv, num_splits=splits)
    ws = torch.empty(fa.fa_decode_workspace_bytes(B, H, d, splits), dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(q)
    lse = torch.empty(B, H, device="cuda")
    fa.fa_decode_ex(q, Kc, Vc, o2, Lkv, ws, lse_out=lse, num_splits=splits)
    torch.cuda.synchronize()
    c = _decode_compare(q, Kc, Vc, o, lengths)
    c2 = _decode_compare(q, Kc, Vc, o2, lengths, lse=lse)
    assert c.ok() and c2.ok(), (c, c2)
    assert torch.all(o[3] == 0)  # empty cache -> o = 0


def test_decode_padded_layout_and_scale():
    fa = _fa()
    _say("decode padded")
    B, H, d, cap = 3, 4, 128, 1500
    lengths = np.array([1500, 7, 777], dtype=np.int64)
    q = synth.torch_normal(510, (B, H, d), "cuda")
    Kc = synth.torch_normal(511, (B, H, cap, d), "cuda")
    Vc = synth.torch_normal(512, (B, H, cap, d), "cuda")
    Lkv = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(B, H, device="cuda")
    ws = torch.empty(fa.fa_decode_workspace_bytes(B, H, d, 5), dtype=torch.uint8, device="cuda")
    fa.fa_decode_ex(q, Kc, Vc, o, Lkv, ws, lse_out=lse, kv_seq_capacity=cap, num_splits=5, scale=0.3)
    torch.cuda.synchronize()
    c = _decode_compare(q, Kc, Vc, o, lengths, lse=lse, scale=0.3, capacity=cap)
    assert c.ok(), c


def test_decode_split_invariance_and_prefill_row():
    """The merge is order-free ('Infra: Flash Attention', Prefill and
    decode): any split count gives the same answer within rounding; and the
    decode of a query equals that query's row of non-causal prefill."""
    fa = _fa()
    _say("decode split invariance")
    B, H, N, d = 1, 2, 2048, 128
    Q, K, V = (synth.torch_normal(520 + t, (B, H, N, d), "cuda") for t in range(3))
    O = torch.empty_like(Q)
    L = torch.empty(B, H, N, device="cuda")
    fa.fa_fwd(Q, K, V, O, L, causal=False)
    Lkv = torch.full((B,), N, dtype=torch.int32, device="cuda")
    q = Q[:, :, 100].contiguous()
    outs = []
    for s in (1, 2, 5, 32, 0):
        o = torch.empty_like(q)
        fa.fa_decode(q, K, V, o, Lkv, num_splits=s)
        outs.append(o)
    torch.cuda.synchronize()
    for o in outs:
        assert float((o.float() - outs[0].float()).abs().max()) <= 2 * BF16_O
        assert float((o.float() - O[:, :, 100].float()).abs().max()) <= 2 * BF16_O
    c = _decode_compare(q, K, V, outs[-1], np.array([N]))
    assert c.ok(), c


def test_decode_32k_workload_all_heads():
    fa = _fa()
    cfg = synth.WORKLOADS["decode_32k"]
    _say("decode_32k", cfg)
    q, Kc, Vc, lengths = synth.decode_inputs("decode_32k", "cuda")
    Lkv = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    fa.fa_decode(q, Kc, Vc, o, Lkv, num_splits=0)
    B, H, d = q.shape
    ws = torch.empty(fa.fa_decode_workspace_bytes(B, H, d, 64), dtype=torch.uint8, device="cuda")
    o64 = torch.empty_like(q)
    lse = torch.empty(B, H, device="cuda")
    fa.fa_decode_ex(q, Kc, Vc, o64, Lkv, ws, lse_out=lse, num_splits=64)
    torch.cuda.synchronize()
    c = _decode_compare(q, Kc, Vc, o, lengths)
    c64 = _decode_compare(q, Kc, Vc, o64, lengths, lse=lse)
    print("decode_32k auto:", c, "| 64 splits:", c64)
    assert c.ok() and c64.ok(), (c, c64)


def test_decode_varlen_workload_all_pairs():
    fa = _fa()
    cfg = synth.WORKLOADS["decode_varlen"]
    q, Kc, Vc, lengths = synth.decode_inputs("decode_varlen", "cuda")
    _say("decode_varlen", cfg, "lengths", lengths.tolist())
    Lkv = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    fa.fa_decode(q, Kc, Vc, o, Lkv, num_splits=0)
    B, H, d = q.shape
    ws = torch.empty(fa.fa_decode_workspace_bytes(B, H, d, 0), dtype=torch.uint8, device="cuda")
    lse = torch.empty(B, H, device="cuda")
    o2 = torch.empty_like(q)
    fa.fa_decode_ex(q, Kc, Vc, o2, Lkv, ws, lse_out=lse, num_splits=0)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    c = _decode_compare(q, Kc, Vc, o2, lengths, lse=lse)
    print("decode_varlen (all 256 pairs)", c)
    assert c.n == q.numel()
    assert c.ok(), c
    assert torch.isfinite(o.float()).all()


# --------------------------------------------------------------------------
# larger than the workloads: long sequences, many heads, long caches
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_bf16_long_sequence_sampled(causal):
    """N = 65536 (256 query tiles, 1024 KV tiles per head), sampled rows."""
    fa = _fa()
    _say("bf16 N=65536", causal)
    shape = (1, 2, 65536, 128)
    Q, K, V = (synth.torch_normal(900 + t, shape, "cuda", "bf16") for t in range(3))
    O = torch.empty_like(Q)
    L = torch.empty(shape[:3], device="cuda")
    fa.fa_fwd(Q, K, V, O, L, causal=causal)
    torch.cuda.synchronize()
    rows = _rows_sample(shape[2], 3)
    c = _prefill_compare(Q, K, V, O, L, 1 / math.sqrt(128), causal, rows=rows, heads=[(0, 0), (0, 1)])
    print(f"N=65536 causal={causal}", c)
    assert c.ok(), c


@pytest.mark.parametrize("causal", [False, True])
def test_bf16_many_heads_sampled(causal):
    """B = 16, H = 128: 2048 heads, several units per persistent workgroup
    (causal) or eight query tiles per head spread over the XCDs."""
    fa = _fa()
    _say("bf16 2048 heads", causal)
    shape = (16, 128, 1000, 64)
    Q, K, V = (synth.torch_normal(910 + t, shape, "cuda", "bf16") for t in range(3))
    O = torch.empty_like(Q)
    L = torch.empty(shape[:3], device="cuda")
    fa.fa_fwd(Q, K, V, O, L, causal=causal)
    torch.cuda.synchronize()
    heads = [(0, 0), (3, 77), (9, 1), (15, 127)]
    c = _prefill_compare(Q, K, V, O, L, 1 / math.sqrt(64), causal, heads=heads)
    assert c.ok(), c
    assert torch.isfinite(O).all() and torch.isfinite(L).all()


@pytest.mark.parametrize("splits", [0, 256])
def test_decode_million_token_cache(splits):
    """One query against 2^20 cached keys per head."""
    fa = _fa()
    _say("decode L=2^20", splits)
    B, H, Lc, d = 1, 2, 1 << 20, 128
    q = synth.torch_normal(920, (B, H, d), "cuda")
    Kc = synth.torch_normal(921, (B, H, Lc, d), "cuda")
    Vc = synth.torch_normal(922, (B, H, Lc, d), "cuda")
    lengths = np.array([Lc], dtype=np.int64)
    Lkv = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    fa.fa_decode(q, Kc, Vc, o, Lkv, num_splits=splits)
    torch.cuda.synchronize()
    c = _decode_compare(q, Kc, Vc, o, lengths)
    print(f"decode L=2^20 splits={splits}", c)
    assert c.ok(), c
