"""The two measurement kernels behind the bench's measured ceilings, through
the C ABI: the HBM read probe reads every word of its buffer (and nothing
else), the MFMA probe computes the products it claims and its stamps give a
plausible clock."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9  # the one folded value the read probe stores


def _fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_02_amd as fa

    return fa


@pytest.mark.parametrize("where", ["first", "unrolled", "tail", "last"])
def test_hbm_read_probe_reads_every_word(where):
    """A buffer of zeros with one word (MAGIC, 0, 0, 0): exactly the thread
    that reads that word folds MAGIC and stores it, into the slot of its
    workgroup; the size leaves a ragged tail after the unrolled loop."""
    fa = _fa()
    wg = 3
    stride = wg * 256
    n16 = 16 * stride + 37     # two passes of the 8-load loop, then a tail
    w = {"first": 0, "unrolled": 13 * stride + 301, "tail": 16 * stride + 11, "last": n16 - 1}[where]
    print("[case] hbm probe", where, "word", w, flush=True)
    host = np.zeros(4 * n16, dtype=np.uint32)
    host[4 * w] = MAGIC
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((wg,), 7, dtype=torch.int32, device="cuda")
    fa.fa_probe_hbm_read(buf, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    want = np.full(wg, 7, dtype=np.uint32)
    want[(w % stride) // 256] = MAGIC
    assert np.array_equal(got, want), (got, want)


def _bf16(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).double().numpy()


def test_mfma_probe_products_and_clock():
    """Per wavefront, the 64 lanes' stored sums add up to 4 chains x iters x
    the sum of the 32x32 product of the operands the kernel builds (lane l of
    half h = l / 32 holds row (column) l mod 32 of A (B) at the 8 k-slots of
    that half), whatever the order of k inside a half."""
    fa = _fa()
    wg, iters = 3, 5
    sink = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
    stamps = torch.zeros(wg, 2, dtype=torch.int64, device="cuda")
    fa.fa_probe_mfma_bf16(wg, iters, sink, stamps)
    torch.cuda.synchronize()
    lanes = np.arange(64)
    a = np.array([[0.001 * ((l + k) & 7) for k in range(8)] for l in lanes])
    b = np.array([[0.002 * ((3 * l + k) & 7) for k in range(8)] for l in lanes])
    a, b = _bf16(a), _bf16(b)
    total = sum(a[32 * h:32 * h + 32, k].sum() * b[32 * h:32 * h + 32, k].sum() for h in range(2) for k in range(8))
    want = 4 * iters * total
    got = sink.cpu().double().numpy().reshape(-1, 64).sum(1)
    assert np.allclose(got, want, rtol=1e-4), (got[:4], want)
    assert (stamps.cpu()[:, 0] > 0).all()

    # a longer loop: the stamps give the clock the wavefronts ran at
    wg, iters = 4, 20000
    sink = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
    stamps = torch.zeros(wg, 2, dtype=torch.int64, device="cuda")
    fa.fa_probe_mfma_bf16(wg, iters, sink, stamps)
    torch.cuda.synchronize()
    st = stamps.cpu().double().numpy()
    assert (st[:, 0] >= iters * 4 * 32).all(), st      # at least 32 clk per 32x32x16 MFMA
    ghz = st[:, 0] / (st[:, 1] / 1e8) / 1e9
    print("[case] mfma probe clock GHz", ghz, flush=True)
    assert ((ghz > 0.3) & (ghz < 3.0)).all(), ghz


def _hash(x):
    x = x.astype(np.uint64) & 0xFFFFFFFF
    x ^= x >> 16
    x = (x * 0x7FEB352D) & 0xFFFFFFFF
    x ^= x >> 15
    x = (x * 0x846CA68B) & 0xFFFFFFFF
    x ^= x >> 16
    return x


def test_mfma_mixed_probe_products():
    """The mixed-operand probe: per wavefront the stored sums add up to iters
    x the sum over its four chains of the 32x32 products of the operands the
    kernel hashes (rebuilt here with the same integer hash, rounded to bf16),
    and a different seed gives different operands."""
    fa = _fa()
    wg, iters, seed = 2, 3, 7
    sink = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
    stamps = torch.zeros(wg, 2, dtype=torch.int64, device="cuda")
    fa.fa_probe_mfma_bf16_mixed(wg, iters, sink, stamps, seed=seed)
    torch.cuda.synchronize()
    got = sink.cpu().double().numpy().reshape(-1, 64).sum(1)
    want = []
    for blk in range(wg):
        for w in range(4):
            tid = np.arange(64) + 64 * w
            tot = 0.0
            for c in range(4):
                base = ((seed * 0x9E3779B9) & 0xFFFFFFFF) ^ (((blk * 256 + tid) * 64 + c * 16)[:, None] + np.arange(8))
                ha = _hash((2 * base) & 0xFFFFFFFF)
                hb = _hash((2 * base + 1) & 0xFFFFFFFF)
                a = _bf16((ha >> 8).astype(np.float64) * 2.0 ** -22 - 2.0)
                b = _bf16((hb >> 8).astype(np.float64) * 2.0 ** -22 - 2.0)
                tot += sum(a[32 * h:32 * h + 32, k].sum() * b[32 * h:32 * h + 32, k].sum()
                           for h in range(2) for k in range(8))
            want.append(iters * tot)
    want = np.array(want)
    assert np.allclose(got, want, rtol=1e-3, atol=1e-2 * np.abs(want).max()), (got[:4], want[:4])
    fa.fa_probe_mfma_bf16_mixed(wg, iters, sink, stamps, seed=seed + 1)
    torch.cuda.synchronize()
    assert not np.allclose(sink.cpu().double().numpy().reshape(-1, 64).sum(1), got)
