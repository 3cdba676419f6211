"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, rejects invalid arguments before any HIP call, and plans
launches whose geometry matches the oracle's tile accounting."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _fa():
    import exact_io_aware_02_amd as fa

    return fa


def _header_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\**(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_symbols_exported():
    fa = _fa()
    names = _header_functions()
    assert len(names) >= 12, names
    assert sorted(fa.EXPORTED) == names
    for n in names:
        assert hasattr(fa.lib, n), n


def test_status_strings():
    fa = _fa()
    assert fa.status_string(0) == "ok"
    for s in (-1, -2, -3, -4, -5):
        assert fa.status_string(s) not in ("", "unknown status")
    assert fa.status_string(7) == "unknown status"


A = 1 << 20  # a 16-byte-aligned fake address; only used where validation rejects first


def _fwd(fn, Q=A, K=2 * A, V=3 * A, O=4 * A, L=None, B=1, H=1, N=16, d=64, causal=0, scale=0.125):
    lib = _fa().lib
    return getattr(lib, fn)(Q, K, V, O, L, B, H, N, d, causal, ctypes.c_float(scale), None)


@pytest.mark.parametrize("fn", ["fa_fwd", "fa_fwd_f32"])
@pytest.mark.parametrize(
    "kw,status,msg",
    [
        (dict(Q=None), -1, "null"),
        (dict(O=None), -1, "null"),
        (dict(B=0), -1, ">= 1"),
        (dict(H=-1), -1, ">= 1"),
        (dict(N=0), -1, ">= 1"),
        (dict(d=0), -1, "d must"),
        (dict(d=96), -2, "not supported"),
        (dict(d=256), -2, "not supported"),
        (dict(causal=2), -1, "causal"),
        (dict(scale=0.0), -1, "scale"),
        (dict(scale=-1.0), -1, "scale"),
        (dict(scale=float("inf")), -1, "scale"),
        (dict(scale=float("nan")), -1, "scale"),
        (dict(Q=A + 4), -1, "aligned"),
        (dict(O=A), -1, "overlaps"),
        (dict(O=2 * A + 64), -1, "overlaps"),
        (dict(L=4 * A + 8), -1, "overlaps"),
        (dict(L=5 * A + 2), -1, "aligned"),
        (dict(N=1 << 24, d=128), -1, "2 GiB"),
    ],
)
def test_fwd_rejects_invalid_arguments(fn, kw, status, msg):
    fa = _fa()
    assert _fwd(fn, **kw) == status
    assert msg in fa.last_error()


def _dec(q=A, Kc=2 * A, Vc=3 * A, o=4 * A, B=1, H=1, Lkv=5 * A, d=64, splits=0):
    return _fa().lib.fa_decode(q, Kc, Vc, o, B, H, Lkv, d, splits, None)


@pytest.mark.parametrize(
    "kw,status,msg",
    [
        (dict(q=None), -1, "null"),
        (dict(Lkv=None), -1, "null"),
        (dict(B=0), -1, ">= 1"),
        (dict(H=70000), -1, "65535"),
        (dict(d=100), -2, "not supported"),
        (dict(splits=-1), -1, "num_splits"),
        (dict(splits=5000), -1, "num_splits"),
        (dict(Kc=2 * A + 8), -1, "aligned"),
        (dict(Lkv=5 * A + 2), -1, "misaligned"),
        (dict(o=A), -1, "overlaps"),
    ],
)
def test_decode_rejects_invalid_arguments(kw, status, msg):
    fa = _fa()
    assert _dec(**kw) == status
    assert msg in fa.last_error()


def test_decode_ex_rejects_bad_workspace_and_capacity():
    fa = _fa()
    lib = fa.lib
    args = (A, 2 * A, 3 * A, 4 * A, None, 2, 4, 5 * A)
    # negative capacity
    assert lib.fa_decode_ex(*args, -1, 128, 8, ctypes.c_float(0.1), 6 * A, 1 << 20, None) == -1
    # bad scale
    assert lib.fa_decode_ex(*args, 0, 128, 8, ctypes.c_float(0.0), 6 * A, 1 << 20, None) == -1
    # missing workspace
    assert lib.fa_decode_ex(*args, 0, 128, 8, ctypes.c_float(0.1), None, 1 << 20, None) == -5
    # misaligned workspace
    assert lib.fa_decode_ex(*args, 0, 128, 8, ctypes.c_float(0.1), 6 * A + 16, 1 << 20, None) == -5
    # too small (explicit split count: no device query needed)
    need = 2 * 4 * 8 * 128 * 4 + 256
    assert lib.fa_decode_ex(*args, 0, 128, 8, ctypes.c_float(0.1), 6 * A, need - 1, None) == -5
    assert "too small" in fa.last_error()


def test_decode_noalloc_rejects_before_any_hip_call():
    """The allocation-free decode validates like fa_decode_ex and rejects a
    request whose partials exceed its static scratch, all on the host (an
    explicit split count needs no device query)."""
    fa = _fa()
    lib = fa.lib
    assert lib.fa_decode_noalloc_scratch_bytes() == 4 << 20
    args = (A, 2 * A, 3 * A, 4 * A, None)
    ok = (2, 4, 5 * A, 0, 128)
    assert lib.fa_decode_noalloc(None, *args[1:], *ok, 8, ctypes.c_float(0.1), None) == -1
    assert lib.fa_decode_noalloc(*args, *ok, 8, ctypes.c_float(0.0), None) == -1
    assert lib.fa_decode_noalloc(*args, 2, 4, 5 * A, 0, 100, 8, ctypes.c_float(0.1), None) == -2
    # 64 x 64 x 64 partials of 129 floats: far above 4 MiB
    assert lib.fa_decode_noalloc(*args, 64, 64, 5 * A, 0, 128, 64, ctypes.c_float(0.1), None) == -5
    assert "scratch" in fa.last_error()
    # the largest request that fits at d = 128: 8128 partials
    assert fa.fa_decode_workspace_bytes(8128, 1, 128, 1) <= 4 << 20 < fa.fa_decode_workspace_bytes(8129, 1, 128, 1)


def test_decode_workspace_formula():
    fa = _fa()
    for B, H, d, S in [(1, 32, 128, 64), (8, 32, 128, 8), (3, 5, 64, 7)]:
        parts = B * H * S
        a256 = lambda x: (x + 255) // 256 * 256
        assert fa.fa_decode_workspace_bytes(B, H, d, S) == a256(parts * d * 4) + a256(parts * 4)
        p = fa.fa_decode_plan(B, H, d, S)
        assert p["num_splits"] == S and p["split_workgroups"] == B * H * S
        assert p["workspace_bytes"] == fa.fa_decode_workspace_bytes(B, H, d, S)
    assert fa.fa_decode_workspace_bytes(0, 1, 128, 1) == 0
    # automatic split count, planned for a 256-CU device: cover every CU once,
    # with at least 8 chunks per sequence
    assert fa.fa_decode_plan(1, 32, 128, 0)["num_splits"] == 8
    assert fa.fa_decode_plan(8, 32, 128, 0)["num_splits"] == 8
    assert fa.fa_decode_plan(1, 4, 128, 0)["num_splits"] == 64
    assert fa.fa_decode_plan(1, 1, 128, 0)["num_splits"] == 256


@pytest.mark.parametrize("L", [1, 63, 64, 65, 511, 512, 4096, 32768, 65536, 40001])
@pytest.mark.parametrize("S", [1, 2, 3, 7, 64, 256])
def test_decode_chunks_cover_every_key_once(L, S):
    fa = _fa()
    c = fa.fa_decode_chunk_tokens(L, S)
    assert c % 64 == 0 and c >= 64
    covered = np.zeros(L, dtype=np.int64)
    for s in range(S):
        a, b = s * c, min(L, (s + 1) * c)
        if a < b:
            covered[a:b] += 1
    assert np.all(covered == 1)
    assert fa.fa_decode_chunk_tokens(0, S) == 0


@pytest.mark.parametrize("causal", [0, 1])
@pytest.mark.parametrize("N", [1, 64, 100, 128, 129, 1000, 2048])
def test_fwd_plan_tile_count_matches_oracle(N, causal):
    """The tiles fa_fwd visits are those of Algorithm 1 with the kernel's
    B_r, B_c and whole-tile causal skipping, as counted by the oracle."""
    fa = _fa()
    p = fa.fa_fwd_plan(2, 3, N, 128, causal)
    rng = np.random.default_rng(0)
    Q, K, V = (rng.standard_normal((N, 2)) for _ in range(3))
    _, _, cnt = oracle.tiled_ref(Q, K, V, p["block_rows"], p["block_cols"], 1.0, causal=bool(causal), count=True)
    assert p["tiles_visited"] == 6 * cnt["tiles"]
    q_tiles = -(-N // p["block_rows"])
    assert p["q_tiles"] == q_tiles
    # persistent grid over work units (query tiles, or causal pairs of them),
    # one workgroup per compute unit at most: at d = 128 both kernels are
    # persistent
    assert p["work_units"] == 6 * (-(-q_tiles // 2) if causal else q_tiles)
    assert p["workgroups"] == min(p["work_units"], 256)
    p64 = fa.fa_fwd_plan(2, 3, N, 64, causal)
    assert p64["workgroups"] == (min(p64["work_units"], 256) if causal else p64["work_units"])


def test_fwd_plan_causal_pin_exercise4():
    """With square tiles the causal count is T(T+1)/2 ('CMU 10-423 Lecture
    18', Exercise 4); with B_r = r B_c each query tile covers r KV tiles per
    query-tile step, so the count is r * T(T+1)/2 with T = N / B_r."""
    fa = _fa()
    N = 4096
    p = fa.fa_fwd_plan(1, 1, N, 128, 1)
    r = p["block_rows"] // p["block_cols"]
    T = N // p["block_rows"]
    assert p["tiles_visited"] == r * oracle.causal_tile_count(T)
    assert fa.fa_fwd_plan(1, 1, N, 128, 0)["tiles_visited"] == T * (N // p["block_cols"])


def test_fwd_causal_pairs_balance_work():
    """Each causal work unit pairs query tile p with q_tiles-1-p, so every
    unit visits the same number of KV tiles (q_tiles + 1 tiles of B_r rows'
    worth when q_tiles is even); the units cover every query tile once."""
    fa = _fa()
    N = 4096
    p = fa.fa_fwd_plan(1, 1, N, 128, 1)
    T, r = p["q_tiles"], p["block_rows"] // p["block_cols"]
    per_tile = [r * (qt + 1) for qt in range(T)]  # KV tiles visited by query tile qt
    units = [(q, T - 1 - q) for q in range((T + 1) // 2)]
    covered = sorted(q for u in units for q in set(u))
    assert covered == list(range(T))
    work = {per_tile[a] + (per_tile[b] if b != a else 0) for a, b in units}
    assert work == {r * (T + 1)}
    assert p["work_units"] == len(units)
    assert p["tiles_visited"] == sum(per_tile)


def _paged(q=A, Kp=2 * A, Vp=3 * A, o=4 * A, lse=None, B=2, H=4, table=5 * A, max_blocks=64, Lkv=6 * A,
           num_blocks=100, bs=16, d=128, splits=8, scale=0.1, ws=None, ws_bytes=0):
    return _fa().lib.fa_decode_paged(q, Kp, Vp, o, lse, B, H, table, max_blocks, Lkv, num_blocks, bs, d,
                                     splits, ctypes.c_float(scale), ws, ws_bytes, None)


@pytest.mark.parametrize(
    "kw,status,msg",
    [
        (dict(table=None), -1, "block_table"),
        (dict(table=5 * A + 2), -1, "block_table misaligned"),
        (dict(bs=8), -1, "power of two"),
        (dict(bs=48), -1, "power of two"),
        (dict(bs=0), -1, "power of two"),
        (dict(max_blocks=0), -1, ">= 1"),
        (dict(num_blocks=0), -1, ">= 1"),
        (dict(d=96), -2, "not supported"),
        (dict(splits=-1), -1, "num_splits"),
        (dict(scale=0.0), -1, "scale"),
        (dict(max_blocks=100000, splits=8), -2, "more splits"),
        (dict(ws=7 * A + 16, ws_bytes=1 << 20), -5, "aligned"),
        (dict(ws=7 * A, ws_bytes=16), -5, "too small"),
        (dict(ws=None, ws_bytes=64), -5, "nonzero"),
        (dict(o=5 * A), -1, "overlaps"),
    ],
)
def test_decode_paged_rejects_invalid_arguments(kw, status, msg):
    fa = _fa()
    assert _paged(**kw) == status
    assert msg in fa.last_error()


def test_decode_paged_split_count():
    """Automatic splits follow fa_decode's rule (planned for 256 compute
    units without a device) and are raised until no chunk of the longest
    possible sequence spans more than 2048 blocks."""
    fa = _fa()
    assert fa.fa_decode_paged_splits(1, 32, 2048, 16, 0) == 8
    s = fa.fa_decode_paged_splits(1, 32, 100000, 16, 0)
    assert s > 8
    chunk = fa.fa_decode_chunk_tokens(100000 * 16, s)
    assert -(-chunk // 16) + 1 <= 2048
    assert -(-fa.fa_decode_chunk_tokens(100000 * 16, s // 2) // 16) + 1 > 2048
    assert fa.fa_decode_paged_splits(1, 32, 100000, 16, 8) == 0
    assert fa.fa_decode_paged_splits(1, 32, 64, 12, 8) == 0
    assert fa.fa_decode_paged_splits(2, 4, 64, 16, 5) == 5


def _bwd(Q=A, K=2 * A, V=3 * A, O=4 * A, dO=5 * A, L=6 * A, dQ=7 * A, dK=8 * A, dV=9 * A, B=1, H=1, N=16, d=64,
         causal=0, scale=0.125, ws=None, ws_bytes=0):
    lib = _fa().lib
    return lib.fa_bwd(Q, K, V, O, dO, L, dQ, dK, dV, B, H, N, d, causal, ctypes.c_float(scale), ws, ws_bytes, None)


@pytest.mark.parametrize(
    "kw,status,msg",
    [
        (dict(Q=None), -1, "null"),
        (dict(dO=None), -1, "null"),
        (dict(L=None), -1, "null"),
        (dict(dV=None), -1, "null"),
        (dict(B=0), -1, ">= 1"),
        (dict(N=0), -1, ">= 1"),
        (dict(d=96), -2, "not supported"),
        (dict(causal=3), -1, "causal"),
        (dict(scale=float("nan")), -1, "scale"),
        (dict(dK=8 * A + 8), -1, "aligned"),
        (dict(L=6 * A + 2), -1, "aligned"),
        (dict(dQ=A + 256), -1, "overlap an input"),
        (dict(dV=6 * A), -1, "overlap L"),
        (dict(dK=7 * A + 1024), -1, "each other"),
        (dict(ws=10 * A + 64, ws_bytes=1 << 20), -5, "aligned"),
        (dict(ws=10 * A, ws_bytes=16), -5, "too small"),
        (dict(ws=None, ws_bytes=16), -5, "nonzero"),
        (dict(ws=9 * A, ws_bytes=1 << 20), -1, "overlaps"),
        (dict(N=1 << 24, d=128), -1, "2 GiB"),
        (dict(B=1 << 16, H=1 << 16, N=64), -1, "grid too large"),
    ],
)
def test_bwd_rejects_invalid_arguments(kw, status, msg):
    """Every argument is checked on the host before any HIP call."""
    fa = _fa()
    assert _bwd(**kw) == status
    assert msg in fa.last_error()


def test_bwd_workspace_formula():
    fa = _fa()
    for B, H, N in ((1, 1, 1), (2, 3, 100), (1, 32, 8192)):
        assert fa.fa_bwd_workspace_bytes(B, H, N) == 2 * (-(-(B * H * N * 4) // 256) * 256)
    assert fa.fa_bwd_workspace_bytes(0, 1, 1) == 0


def test_probes_reject_invalid_arguments():
    """The measurement kernels check their buffers and sizes on the host."""
    fa = _fa()
    lib = fa.lib
    assert lib.fa_probe_hbm_read(None, 1024, 4, A, None) == -1
    assert lib.fa_probe_hbm_read(A, 1000, 4, 2 * A, None) == -1          # not a multiple of 16
    assert lib.fa_probe_hbm_read(A + 8, 1024, 4, 2 * A, None) == -1      # misaligned
    assert lib.fa_probe_hbm_read(A, 1024, 0, 2 * A, None) == -1
    assert lib.fa_probe_hbm_read(A, 1024, 4, A + 512, None) == -1        # sink inside buf
    assert "overlaps" in fa.last_error()
    assert lib.fa_probe_mfma_bf16(4, 10, None, None, None) == -1
    assert lib.fa_probe_mfma_bf16(0, 10, A, None, None) == -1
    assert lib.fa_probe_mfma_bf16(4, 0, A, None, None) == -1
    assert lib.fa_probe_mfma_bf16(4, 10, A, A + 4, None) == -1           # stamps misaligned
    assert lib.fa_probe_mfma_bf16(4, 10, A, A + 8, None) == -1           # stamps inside sink
    assert lib.fa_probe_mfma_bf16_mixed(4, 10, 1, None, None, None) == -1
    assert lib.fa_probe_mfma_bf16_mixed(0, 10, 1, A, None, None) == -1
    assert lib.fa_probe_mfma_bf16_mixed(4, 1 << 25, 1, A, None, None) == -1
    assert lib.fa_probe_mfma_bf16_mixed(4, 10, 1, A, A + 8, None) == -1


def test_exp2_poly_share_is_validated():
    """fa_set_fwd_exp2_poly takes 0, 4, 8 or 16 exponentials per 64 and
    leaves the setting unchanged on any other value."""
    fa = _fa()
    lib = fa.lib
    assert lib.fa_get_fwd_exp2_poly() == 0
    try:
        for v in (4, 8, 16, 0):
            assert lib.fa_set_fwd_exp2_poly(v) == 0
            assert lib.fa_get_fwd_exp2_poly() == v
        assert lib.fa_set_fwd_exp2_poly(8) == 0
        for v in (-1, 1, 2, 3, 12, 32, 64):
            assert lib.fa_set_fwd_exp2_poly(v) == -1
            assert lib.fa_get_fwd_exp2_poly() == 8
        assert "0, 4, 8 or 16" in fa.last_error()
    finally:
        lib.fa_set_fwd_exp2_poly(0)


def test_decode_fused_rejects_bad_workspace_and_arguments():
    """The one-launch decode validates like fa_decode_ex; its workspace puts a
    fixed region of 65536 int32 counters before the partials, and B * H above
    65536 is unsupported."""
    fa = _fa()
    lib = fa.lib
    args = (A, 2 * A, 3 * A, 4 * A, None, 2, 4, 5 * A)
    parts = fa.fa_decode_workspace_bytes(2, 4, 128, 8)
    need = fa.fa_decode_fused_workspace_bytes(2, 4, 128, 8)
    assert need == parts + (1 << 18)
    assert fa.fa_decode_fused_workspace_bytes(3, 100, 64, 7) == fa.fa_decode_workspace_bytes(3, 100, 64, 7) + (1 << 18)
    assert fa.fa_decode_fused_workspace_bytes(0, 4, 128, 8) == 0
    assert fa.fa_decode_fused_workspace_bytes(2, 4, 100, 8) == 0
    assert fa.fa_decode_fused_workspace_bytes(257, 256, 128, 1) == 0
    assert fa.fa_decode_fused_workspace_bytes(256, 256, 128, 1) > 0
    G = 1 << 30  # addresses far enough apart for B * H = 65792 rows of q and o
    assert lib.fa_decode_fused(G, 2 * G, 3 * G, 4 * G, None, 257, 256, 5 * G, 0, 128, 1, ctypes.c_float(0.1),
                               6 * G, 1 << 30, None) == -2
    assert "65536" in fa.last_error()
    assert lib.fa_decode_fused(*args, -1, 128, 8, ctypes.c_float(0.1), 6 * A, need, None) == -1
    assert lib.fa_decode_fused(*args, 0, 128, 8, ctypes.c_float(0.0), 6 * A, need, None) == -1
    assert lib.fa_decode_fused(*args, 0, 100, 8, ctypes.c_float(0.1), 6 * A, need, None) == -2
    assert lib.fa_decode_fused(*args, 0, 128, 8, ctypes.c_float(0.1), None, need, None) == -5
    assert lib.fa_decode_fused(*args, 0, 128, 8, ctypes.c_float(0.1), 6 * A + 16, need, None) == -5
    # room for the partials but not the counters
    assert lib.fa_decode_fused(*args, 0, 128, 8, ctypes.c_float(0.1), 6 * A, parts, None) == -5
    assert "too small" in fa.last_error()
    # workspace over o (4 * A, 2 * 4 * 128 bf16) or over lse_out
    assert lib.fa_decode_fused(*args, 0, 128, 8, ctypes.c_float(0.1), 4 * A - 256, need, None) == -1
    assert "overlaps" in fa.last_error()
    argsl = (A, 2 * A, 3 * A, 4 * A, 8 * A + 512, 2, 4, 5 * A)
    assert lib.fa_decode_fused(*argsl, 0, 128, 8, ctypes.c_float(0.1), 8 * A, need, None) == -1
    assert "lse_out" in fa.last_error()
