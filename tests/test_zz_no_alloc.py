"""fa_decode_noalloc (partials in the library's static per-device scratch)
against fa_decode_ex (partials in a caller workspace), through the C ABI.

Both run the same split and combine kernels with the same split count, so the
outputs and log-sum-exps must agree bit for bit.  Two calls in a row, the
second smaller, check that the second call is not disturbed by what the first
left in the scratch; a request larger than the scratch is rejected before
anything is enqueued.
"""

import ctypes
import math

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_02_amd as fa

    return fa


def _inputs(lengths, H, d, seed):
    B = len(lengths)
    total = int(np.sum(lengths)) * H * d
    q = synth.torch_normal(seed, (B, H, d), "cuda", vscale=2.0)
    Kc = synth.torch_normal(seed + 1, (total,), "cuda", vscale=2.0)
    Vc = synth.torch_normal(seed + 2, (total,), "cuda", vscale=2.0)
    Lkv = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    return q, Kc, Vc, Lkv


def _run_pair(fa, lengths, H, d, splits, seed):
    """(o, lse) of fa_decode_noalloc and of fa_decode_ex, raw C calls on the
    current stream."""
    q, Kc, Vc, Lkv = _inputs(lengths, H, d, seed)
    B = len(lengths)
    scale = 1.0 / math.sqrt(d)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    o1 = torch.full((B, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    l1 = torch.full((B, H), float("nan"), device="cuda")
    st = fa.lib.fa_decode_noalloc(P(q), P(Kc), P(Vc), P(o1), P(l1), B, H, P(Lkv), 0, d, splits, scale, stream)
    assert st == 0, fa.last_error()
    ws = torch.empty(fa.fa_decode_workspace_bytes(B, H, d, splits), dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    st = fa.lib.fa_decode_ex(P(q), P(Kc), P(Vc), P(o2), P(l2), B, H, P(Lkv), 0, d, splits, scale, P(ws),
                             ws.numel(), stream)
    assert st == 0, fa.last_error()
    torch.cuda.synchronize()
    return o1, l1, o2, l2


def test_noalloc_matches_workspace_decode_twice():
    fa = _fa()
    # first call: 8 sequences x 16 heads, automatic splits
    print("[case] noalloc call 1: B=8 H=16 d=128 auto splits", flush=True)
    o1, l1, o2, l2 = _run_pair(fa, [4100, 1, 0, 777, 20000, 64, 65, 9000], 16, 128, 0, 1200)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.all(o1[2] == 0) and torch.all(torch.isneginf(l1[2]))
    # second call, smaller: fewer sequences, heads and partials; d = 64
    print("[case] noalloc call 2: B=3 H=4 d=64 5 splits", flush=True)
    o1, l1, o2, l2 = _run_pair(fa, [300, 5000, 17], 4, 64, 5, 1300)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()


def test_noalloc_rejects_requests_above_the_scratch():
    fa = _fa()
    cap = fa.fa_decode_noalloc_scratch_bytes()
    assert cap == 4 << 20
    q, Kc, Vc, Lkv = _inputs([1000] * 4, 64, 128, 1400)
    o = torch.empty(4, 64, 128, dtype=torch.bfloat16, device="cuda")
    # 4 x 64 x 64 = 16384 partials of 129 floats: above 4 MiB
    assert fa.fa_decode_workspace_bytes(4, 64, 128, 64) > cap
    with pytest.raises(fa.FAError) as e:
        fa.fa_decode_noalloc(q, Kc, Vc, o, Lkv, num_splits=64)
    assert e.value.status == fa.FA_ERR_WORKSPACE
    # 16 splits fit (4096 partials) and match the workspace path
    lse = torch.empty(4, 64, device="cuda")
    fa.fa_decode_noalloc(q, Kc, Vc, o, Lkv, lse_out=lse, num_splits=16)
    ws = torch.empty(fa.fa_decode_workspace_bytes(4, 64, 128, 16), dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(o)
    lse2 = torch.empty_like(lse)
    fa.fa_decode_ex(q, Kc, Vc, o2, Lkv, ws, lse_out=lse2, num_splits=16)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
