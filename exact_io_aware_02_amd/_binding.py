"""ctypes binding of libfa.so: argument marshalling only.

Every computation runs in the HIP kernels behind the C ABI declared in
include/fa.h.  The raw entry points take integer device pointers exactly like
the C functions; the tensor-taking wrappers of the same names read shapes,
data pointers and the current stream from torch tensors and call them.  There
is no fallback: if libfa.so is missing, importing this module fails.
"""

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# FA_LIBRARY names another build of the same sources (the host-sanitizer
# build of the dispatch code, for instance); the default is the in-tree one.
LIB_PATH = os.environ.get("FA_LIBRARY") or os.path.join(_HERE, "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_HIP = -3
FA_ERR_NOMEM = -4
FA_ERR_WORKSPACE = -5


class FAError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


class fa_fwd_plan_t(ctypes.Structure):
    _fields_ = [
        ("block_rows", ctypes.c_int),
        ("block_cols", ctypes.c_int),
        ("q_tiles", ctypes.c_int),
        ("kv_tiles", ctypes.c_int),
        ("threads_per_workgroup", ctypes.c_int),
        ("lds_bytes", ctypes.c_int),
        ("workgroups", ctypes.c_int64),
        ("tiles_visited", ctypes.c_int64),
        ("tiles_masked", ctypes.c_int64),
        ("work_units", ctypes.c_int64),
    ]


class fa_decode_plan_t(ctypes.Structure):
    _fields_ = [
        ("num_splits", ctypes.c_int),
        ("threads_per_workgroup", ctypes.c_int),
        ("split_workgroups", ctypes.c_int64),
        ("combine_workgroups", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_size_t),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python exact_io_aware_02_amd/build.py` "
            "(or __graft_entry__.build()); there is no non-HIP fallback"
        )
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    sig = {
        "fa_fwd": (I, [P, P, P, P, P, I, I, I, I, I, F, P]),
        "fa_fwd_f32": (I, [P, P, P, P, P, I, I, I, I, I, F, P]),
        "fa_set_fwd_exp2_poly": (I, [I]),
        "fa_get_fwd_exp2_poly": (I, []),
        "fa_decode": (I, [P, P, P, P, I, I, P, I, I, P]),
        "fa_bwd": (I, [P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, P, Z, P]),
        "fa_bwd_workspace_bytes": (Z, [I, I, I]),
        "fa_decode_ex": (I, [P, P, P, P, P, I, I, P, I, I, I, F, P, Z, P]),
        "fa_decode_workspace_bytes": (Z, [I, I, I, I]),
        "fa_decode_fused": (I, [P, P, P, P, P, I, I, P, I, I, I, F, P, Z, P]),
        "fa_decode_fused_workspace_bytes": (Z, [I, I, I, I]),
        "fa_decode_noalloc": (I, [P, P, P, P, P, I, I, P, I, I, I, F, P]),
        "fa_decode_noalloc_scratch_bytes": (Z, []),
        "fa_decode_paged": (I, [P, P, P, P, P, I, I, P, I, P, I, I, I, I, F, P, Z, P]),
        "fa_decode_paged_splits": (I, [I, I, I, I, I]),
        "fa_fwd_plan": (I, [I, I, I, I, I, ctypes.POINTER(fa_fwd_plan_t)]),
        "fa_decode_plan": (I, [I, I, I, I, ctypes.POINTER(fa_decode_plan_t)]),
        "fa_decode_chunk_tokens": (I, [I, I]),
        "fa_release_workspace": (I, []),
        "fa_probe_hbm_read": (I, [P, Z, I, P, P]),
        "fa_probe_mfma_bf16": (I, [I, I, P, P, P]),
        "fa_probe_mfma_bf16_mixed": (I, [I, I, ctypes.c_uint32, P, P, P]),
        "fa_status_string": (ctypes.c_char_p, [I]),
        "fa_last_error": (ctypes.c_char_p, []),
        "fa_version": (I, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()

# names of every symbol include/fa.h declares
EXPORTED = (
    "fa_fwd",
    "fa_fwd_f32",
    "fa_set_fwd_exp2_poly",
    "fa_get_fwd_exp2_poly",
    "fa_bwd",
    "fa_bwd_workspace_bytes",
    "fa_decode",
    "fa_decode_ex",
    "fa_decode_workspace_bytes",
    "fa_decode_fused",
    "fa_decode_fused_workspace_bytes",
    "fa_decode_noalloc",
    "fa_decode_noalloc_scratch_bytes",
    "fa_decode_paged",
    "fa_decode_paged_splits",
    "fa_fwd_plan",
    "fa_decode_plan",
    "fa_decode_chunk_tokens",
    "fa_release_workspace",
    "fa_probe_hbm_read",
    "fa_probe_mfma_bf16",
    "fa_probe_mfma_bf16_mixed",
    "fa_status_string",
    "fa_last_error",
    "fa_version",
)


def _check(status):
    if status != FA_OK:
        msg = lib.fa_last_error().decode() or lib.fa_status_string(status).decode()
        raise FAError(status, msg)
    return status


def last_error():
    return lib.fa_last_error().decode()


def status_string(status):
    return lib.fa_status_string(status).decode()


# --------------------------------------------------------------------------
# host-only planning
# --------------------------------------------------------------------------

def fa_fwd_plan(B, H, N, d, causal):
    p = fa_fwd_plan_t()
    _check(lib.fa_fwd_plan(B, H, N, d, int(causal), ctypes.byref(p)))
    return {f: getattr(p, f) for f, _ in fa_fwd_plan_t._fields_}


def fa_decode_plan(B, H, d, num_splits=0):
    p = fa_decode_plan_t()
    _check(lib.fa_decode_plan(B, H, d, num_splits, ctypes.byref(p)))
    return {f: getattr(p, f) for f, _ in fa_decode_plan_t._fields_}


def fa_decode_chunk_tokens(kv_len, num_splits):
    return lib.fa_decode_chunk_tokens(int(kv_len), int(num_splits))


def fa_decode_workspace_bytes(B, H, d, num_splits=0):
    return lib.fa_decode_workspace_bytes(B, H, d, num_splits)


def fa_release_workspace():
    _check(lib.fa_release_workspace())


# --------------------------------------------------------------------------
# tensor wrappers (torch is used for device memory and the stream only)
# --------------------------------------------------------------------------

def _stream_ptr(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _expect(t, dtype, shape, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")


def fa_fwd(Q, K, V, O, L=None, causal=False, scale=None, stream=None):
    """O = softmax(Q K^T * scale) V for bf16 [B, H, N, d]; L (fp32 [B, H, N])
    receives the per-row log-sum-exp if given."""
    import torch

    B, H, N, d = Q.shape
    for t, n in ((Q, "Q"), (K, "K"), (V, "V"), (O, "O")):
        _expect(t, torch.bfloat16, (B, H, N, d), n)
    if L is not None:
        _expect(L, torch.float32, (B, H, N), "L")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(lib.fa_fwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(L), B, H, N, d, int(causal),
                      float(scale), _stream_ptr(stream)))
    return O, L


def fa_set_fwd_exp2_poly(per64):
    """Exponentials per 64 that the d = 128 bf16 forward evaluates by a
    polynomial on the multiply-add units (0, 4, 8 or 16; 0 is the default).
    Returns the previous setting."""
    prev = lib.fa_get_fwd_exp2_poly()
    _check(lib.fa_set_fwd_exp2_poly(int(per64)))
    return prev


def fa_get_fwd_exp2_poly():
    return lib.fa_get_fwd_exp2_poly()


def fa_bwd_workspace_bytes(B, H, N):
    return lib.fa_bwd_workspace_bytes(int(B), int(H), int(N))


def fa_bwd(Q, K, V, O, dO, L, dQ, dK, dV, causal=False, scale=None, workspace=None, stream=None):
    """Gradients dQ, dK, dV (bf16 [B, H, N, d], overwritten) of the forward
    that produced O and L from Q, K, V, given dO.  workspace: a device tensor
    of at least fa_bwd_workspace_bytes(B, H, N) bytes, or None for the
    library's internal one."""
    import torch

    B, H, N, d = Q.shape
    for t, n in ((Q, "Q"), (K, "K"), (V, "V"), (O, "O"), (dO, "dO"), (dQ, "dQ"), (dK, "dK"), (dV, "dV")):
        _expect(t, torch.bfloat16, (B, H, N, d), n)
    _expect(L, torch.float32, (B, H, N), "L")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws, wsb = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel() * workspace.element_size())
    _check(lib.fa_bwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(L), _ptr(dQ), _ptr(dK), _ptr(dV), B, H, N,
                      d, int(causal), float(scale), ws, wsb, _stream_ptr(stream)))
    return dQ, dK, dV


def fa_fwd_f32(Q, K, V, O, L=None, causal=False, scale=None, stream=None):
    """fp32 variant of fa_fwd: Q, K, V, O fp32 [B, H, N, d]."""
    import torch

    B, H, N, d = Q.shape
    for t, n in ((Q, "Q"), (K, "K"), (V, "V"), (O, "O")):
        _expect(t, torch.float32, (B, H, N, d), n)
    if L is not None:
        _expect(L, torch.float32, (B, H, N), "L")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(lib.fa_fwd_f32(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(L), B, H, N, d, int(causal),
                          float(scale), _stream_ptr(stream)))
    return O, L


def _decode_shapes(q, Kcache, Vcache, o, Lkv):
    import torch

    B, H, d = q.shape
    _expect(q, torch.bfloat16, (B, H, d), "q")
    _expect(o, torch.bfloat16, (B, H, d), "o")
    _expect(Lkv, torch.int32, (B,), "Lkv")
    for t, n in ((Kcache, "Kcache"), (Vcache, "Vcache")):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError(f"{n} must be a contiguous bf16 device tensor")
    return B, H, d


def fa_decode(q, Kcache, Vcache, o, Lkv, num_splits=0, stream=None):
    """Flash-Decoding: q, o bf16 [B, H, d]; Kcache/Vcache packed bf16 caches;
    Lkv int32 [B] device lengths.  Uses the library's internal workspace."""
    B, H, d = _decode_shapes(q, Kcache, Vcache, o, Lkv)
    _check(lib.fa_decode(_ptr(q), _ptr(Kcache), _ptr(Vcache), _ptr(o), B, H, _ptr(Lkv), d,
                         int(num_splits), _stream_ptr(stream)))
    return o


def fa_decode_ex(q, Kcache, Vcache, o, Lkv, workspace, lse_out=None, kv_seq_capacity=0,
                 num_splits=0, scale=None, stream=None):
    """fa_decode with a caller-owned workspace (a device tensor of at least
    fa_decode_workspace_bytes(...) bytes), optional lse_out fp32 [B, H] and
    the padded layout when kv_seq_capacity > 0."""
    import torch

    B, H, d = _decode_shapes(q, Kcache, Vcache, o, Lkv)
    if lse_out is not None:
        _expect(lse_out, torch.float32, (B, H), "lse_out")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.fa_decode_ex(_ptr(q), _ptr(Kcache), _ptr(Vcache), _ptr(o), _ptr(lse_out), B, H,
                            _ptr(Lkv), int(kv_seq_capacity), d, int(num_splits), float(scale),
                            _ptr(workspace), nbytes, _stream_ptr(stream)))
    return o, lse_out


def fa_decode_fused_workspace_bytes(B, H, d, num_splits=0):
    return lib.fa_decode_fused_workspace_bytes(int(B), int(H), int(d), int(num_splits))


def fa_decode_fused(q, Kcache, Vcache, o, Lkv, workspace, lse_out=None, kv_seq_capacity=0, num_splits=0,
                    scale=None, stream=None):
    """fa_decode_ex in one launch (the last split workgroup of each (b, h)
    merges).  workspace: a device tensor of at least
    fa_decode_fused_workspace_bytes(...) bytes whose counters (its last
    B * H int32 after the partials) are zero before the first call, e.g.
    torch.zeros; every completed call leaves them zero."""
    import torch

    B, H, d = _decode_shapes(q, Kcache, Vcache, o, Lkv)
    if lse_out is not None:
        _expect(lse_out, torch.float32, (B, H), "lse_out")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.fa_decode_fused(_ptr(q), _ptr(Kcache), _ptr(Vcache), _ptr(o), _ptr(lse_out), B, H, _ptr(Lkv),
                               int(kv_seq_capacity), d, int(num_splits), float(scale), _ptr(workspace), nbytes,
                               _stream_ptr(stream)))
    return o, lse_out


def fa_decode_noalloc_scratch_bytes():
    return lib.fa_decode_noalloc_scratch_bytes()


def fa_decode_noalloc(q, Kcache, Vcache, o, Lkv, lse_out=None, kv_seq_capacity=0, num_splits=0, scale=None,
                      stream=None):
    """fa_decode_ex with the partials in the library's static per-device
    scratch: allocates nothing (calls that overlap on one device race)."""
    import torch

    B, H, d = _decode_shapes(q, Kcache, Vcache, o, Lkv)
    if lse_out is not None:
        _expect(lse_out, torch.float32, (B, H), "lse_out")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(lib.fa_decode_noalloc(_ptr(q), _ptr(Kcache), _ptr(Vcache), _ptr(o), _ptr(lse_out), B, H, _ptr(Lkv),
                                 int(kv_seq_capacity), d, int(num_splits), float(scale), _stream_ptr(stream)))
    return o, lse_out


def fa_decode_paged_splits(B, H, max_blocks, block_size, num_splits=0):
    """Split count fa_decode_paged uses (0 if the arguments are invalid)."""
    return lib.fa_decode_paged_splits(int(B), int(H), int(max_blocks), int(block_size), int(num_splits))


def fa_decode_paged(q, Kpool, Vpool, o, block_table, Lkv, lse_out=None, num_splits=0, scale=None,
                    workspace=None, stream=None):
    """Flash-Decoding through a block table: q, o bf16 [B, H, d]; Kpool/Vpool
    bf16 [num_blocks, H, block_size, d]; block_table int32 [B, max_blocks];
    Lkv int32 [B]; optional lse_out fp32 [B, H]; workspace a device tensor
    (None = the library's own)."""
    import torch

    B, H, d = q.shape
    _expect(q, torch.bfloat16, (B, H, d), "q")
    _expect(o, torch.bfloat16, (B, H, d), "o")
    _expect(Lkv, torch.int32, (B,), "Lkv")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B \
            or not block_table.is_contiguous() or block_table.device.type != "cuda":
        raise ValueError("block_table must be a contiguous int32 device tensor [B, max_blocks]")
    for t_, n in ((Kpool, "Kpool"), (Vpool, "Vpool")):
        if t_.dtype != torch.bfloat16 or t_.dim() != 4 or not t_.is_contiguous() or t_.device.type != "cuda" \
                or t_.shape[1] != H or t_.shape[3] != d:
            raise ValueError(f"{n} must be a contiguous bf16 device tensor [num_blocks, H, block_size, d]")
    if Kpool.shape != Vpool.shape:
        raise ValueError("Kpool and Vpool must have the same shape")
    num_blocks, _, block_size, _ = Kpool.shape
    if lse_out is not None:
        _expect(lse_out, torch.float32, (B, H), "lse_out")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.fa_decode_paged(_ptr(q), _ptr(Kpool), _ptr(Vpool), _ptr(o), _ptr(lse_out), B, H,
                               _ptr(block_table), int(block_table.shape[1]), _ptr(Lkv), int(num_blocks),
                               int(block_size), d, int(num_splits), float(scale), _ptr(workspace), nbytes,
                               _stream_ptr(stream)))
    return o, lse_out


# --------------------------------------------------------------------------
# measurement kernels (measured ceilings beside the published peaks)
# --------------------------------------------------------------------------

def fa_probe_hbm_read(buf, sink, workgroups=None, stream=None):
    """Reads every byte of the contiguous device tensor `buf` once; sink is a
    uint32/int32 device tensor of at least `workgroups` elements (default:
    its length)."""
    if workgroups is None:
        workgroups = sink.numel()
    if sink.numel() * sink.element_size() < 4 * workgroups or sink.element_size() != 4:
        raise ValueError("sink must hold one 4-byte word per workgroup")
    for t, n in ((buf, "buf"), (sink, "sink")):
        if not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError(f"{n} must be a contiguous device tensor")
    _check(lib.fa_probe_hbm_read(_ptr(buf), buf.numel() * buf.element_size(), int(workgroups), _ptr(sink),
                                 _stream_ptr(stream)))


def fa_probe_mfma_bf16(workgroups, iters, sink, stamps=None, stream=None):
    """workgroups x 4 wavefronts of iters x 4 bf16 MFMAs (32x32x16); sink
    float32 [workgroups * 256], stamps int64 [workgroups, 2] or None."""
    import torch

    _expect(sink, torch.float32, (workgroups * 256,), "sink")
    if stamps is not None:
        _expect(stamps, torch.int64, (workgroups, 2), "stamps")
    _check(lib.fa_probe_mfma_bf16(int(workgroups), int(iters), _ptr(sink), _ptr(stamps), _stream_ptr(stream)))


def fa_probe_mfma_bf16_mixed(workgroups, iters, sink, stamps=None, seed=1, stream=None):
    """fa_probe_mfma_bf16 with pseudo-random operands that differ between
    consecutive products (seeded by `seed`)."""
    import torch

    _expect(sink, torch.float32, (workgroups * 256,), "sink")
    if stamps is not None:
        _expect(stamps, torch.int64, (workgroups, 2), "stamps")
    _check(lib.fa_probe_mfma_bf16_mixed(int(workgroups), int(iters), int(seed) & 0xFFFFFFFF, _ptr(sink),
                                        _ptr(stamps), _stream_ptr(stream)))
