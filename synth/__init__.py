"""Seeded synthetic inputs shared by the tests, the bench and the oracle.

This module holds no attention arithmetic: only the workload shapes, seeded
normal draws, and rounding of the drawn values to the storage dtype the GPU
path receives (bf16 by round-to-nearest-even, or fp32 as drawn).  The HIP path
and the oracle both consume what it produces; neither is imported here.

Workloads (the shapes of the pages' examples: N = 8192, d = 128 bf16 per head
as in "Infra: Flash Attention", section "GPU memory hierarchy and IO"; decode
of one query against a 32,768-token cache with B = 1, H = 32 as in the airsota
Flash-Decoding card, section 3; long-context decode beyond 16K from its
section 4):

  fp32_small     B=1 H=1  N=256  d=64  fp32 N(0,1), non-causal
  prefill_8k     B=1 H=32 N=8192 d=128 bf16 N(0,1), non-causal
  causal_4k      B=4 H=32 N=4096 d=128 bf16 N(0,1), causal
  decode_32k     B=1 H=32 L=32768 d=128 bf16 N(0,1)
  decode_varlen  B=8 H=32 d=128, L_b uniform on [4096, 65536], bf16 2*N(0,1)
  decode_paged   decode_varlen's shapes and lengths with the cache in blocks
                 of 16 tokens at seeded, scattered physical positions behind a
                 block table (the layout of "CMU 10-423 Lecture 18", section
                 7.3), bf16 2*N(0,1)
"""

import numpy as np

WORKLOADS = {
    "fp32_small": dict(kind="prefill", B=1, H=1, N=256, d=64, dtype="f32", causal=False, vscale=1.0, seed=1),
    "prefill_8k": dict(kind="prefill", B=1, H=32, N=8192, d=128, dtype="bf16", causal=False, vscale=1.0, seed=2),
    "causal_4k": dict(kind="prefill", B=4, H=32, N=4096, d=128, dtype="bf16", causal=True, vscale=1.0, seed=3),
    "decode_32k": dict(kind="decode", B=1, H=32, L=32768, d=128, dtype="bf16", vscale=1.0, seed=4),
    "decode_varlen": dict(kind="decode", B=8, H=32, Lmin=4096, Lmax=65536, d=128, dtype="bf16", vscale=2.0, seed=5),
    "decode_paged": dict(kind="paged", B=8, H=32, Lmin=4096, Lmax=65536, d=128, dtype="bf16", vscale=2.0, seed=6,
                         block_size=16, spare_blocks=64),
}


def varlen_lengths(B=8, lo=4096, hi=65536, seed=5000):
    """Per-sequence KV lengths, uniform integers on [lo, hi]."""
    return np.random.default_rng(seed).integers(lo, hi, endpoint=True, size=B).astype(np.int64)


def bf16_round_np(x):
    """Round float32 values to the nearest bf16 (ties to even); returns the
    rounded values as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(x.shape)


def np_normal(seed, shape, vscale=1.0, dtype="bf16"):
    """Seeded N(0, vscale^2) float32 draw on the host, rounded to bf16 when
    dtype == 'bf16'.  Returns float32 values."""
    x = np.random.default_rng(seed).standard_normal(size=shape, dtype=np.float32)
    if vscale != 1.0:
        x = x * np.float32(vscale)  # power-of-two scales commute with rounding
    return bf16_round_np(x) if dtype == "bf16" else x


def torch_normal(seed, shape, device, dtype="bf16", vscale=1.0):
    """Seeded N(0, vscale^2) draw made on `device` with torch's generator,
    stored as torch.bfloat16 (round-to-nearest-even) or torch.float32."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if vscale != 1.0:
        x.mul_(vscale)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def prefill_inputs(name_or_cfg, device, seed_offset=0):
    """(Q, K, V) torch tensors [B, H, N, d] for a prefill workload."""
    cfg = WORKLOADS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    shape = (cfg["B"], cfg["H"], cfg["N"], cfg["d"])
    base = 1000 * (cfg["seed"] + seed_offset)
    return tuple(
        torch_normal(base + t, shape, device, cfg["dtype"], cfg["vscale"]) for t in range(3)
    )


def decode_inputs(name_or_cfg, device, lengths=None, seed_offset=0):
    """(q [B,H,d], Kcache, Vcache, lengths) for a decode workload.  The caches
    are packed: sequence b occupies [H, L_b, d] and sequences follow each other
    in b order, so the uniform case is plain [B, H, L, d]."""
    cfg = WORKLOADS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    B, H, d = cfg["B"], cfg["H"], cfg["d"]
    if lengths is None:
        if "L" in cfg:
            lengths = np.full((B,), cfg["L"], dtype=np.int64)
        else:
            lengths = varlen_lengths(B, cfg["Lmin"], cfg["Lmax"])
    lengths = np.asarray(lengths, dtype=np.int64)
    total = int(lengths.sum()) * H * d
    base = 1000 * (cfg["seed"] + seed_offset)
    q = torch_normal(base + 0, (B, H, d), device, cfg["dtype"], cfg["vscale"])
    Kc = torch_normal(base + 1, (total,), device, cfg["dtype"], cfg["vscale"])
    Vc = torch_normal(base + 2, (total,), device, cfg["dtype"], cfg["vscale"])
    return q, Kc, Vc, lengths


def packed_offsets(lengths, H, d):
    """Element offset of sequence b's [H, L_b, d] block in a packed cache."""
    lengths = np.asarray(lengths, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(lengths)[:-1]]) * H * d


def block_table(lengths, block_size, spare_blocks=0, seed=0):
    """A seeded block table: (table int32 [B, max_blocks], num_blocks).

    Every physical block id in [0, num_blocks) is dealt once, in the order of
    a seeded permutation, to the sequences' logical blocks (sequence 0 first);
    `spare_blocks` ids stay unused, and entries past a sequence's blocks are
    -1."""
    lengths = np.asarray(lengths, dtype=np.int64)
    nbs = [-(-int(L) // int(block_size)) for L in lengths]
    num_blocks = sum(nbs) + int(spare_blocks)
    perm = np.random.default_rng(seed).permutation(num_blocks)
    table = np.full((len(lengths), max(1, max(nbs) if nbs else 1)), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(nbs):
        table[b, :n] = perm[k:k + n]
        k += n
    return table, num_blocks


def paged_inputs(name_or_cfg, device, lengths=None, block_size=None, spare_blocks=None, seed_offset=0):
    """(q [B,H,d], Kpool, Vpool [num_blocks, H, block_size, d], table int32
    [B, max_blocks], lengths) for a paged decode workload.  Pool slots that
    hold no token are filled with draws too (never read by a correct
    reader)."""
    cfg = WORKLOADS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    B, H, d = cfg["B"], cfg["H"], cfg["d"]
    bs = int(block_size if block_size is not None else cfg["block_size"])
    spare = int(spare_blocks if spare_blocks is not None else cfg.get("spare_blocks", 0))
    if lengths is None:
        if "L" in cfg:
            lengths = np.full((B,), cfg["L"], dtype=np.int64)
        else:
            lengths = varlen_lengths(B, cfg["Lmin"], cfg["Lmax"])
    lengths = np.asarray(lengths, dtype=np.int64)
    base = 1000 * (cfg["seed"] + seed_offset)
    table, num_blocks = block_table(lengths, bs, spare, seed=base + 3)
    q = torch_normal(base + 0, (B, H, d), device, cfg["dtype"], cfg["vscale"])
    Kp = torch_normal(base + 1, (num_blocks, H, bs, d), device, cfg["dtype"], cfg["vscale"])
    Vp = torch_normal(base + 2, (num_blocks, H, bs, d), device, cfg["dtype"], cfg["vscale"])
    return q, Kp, Vp, table, lengths
