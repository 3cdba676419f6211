"""Exact attention forward (FlashAttention), its backward, and Flash-Decoding
for AMD MI355X (gfx950).

The compute lives in libfa.so (HIP kernels behind the C ABI of include/fa.h);
this package is its ctypes binding.  Build the library in-tree with
`python exact_io_aware_02_amd/build.py`.
"""

from ._binding import (  # noqa: F401
    EXPORTED,
    FAError,
    FA_OK,
    FA_ERR_INVALID_ARG,
    FA_ERR_UNSUPPORTED,
    FA_ERR_HIP,
    FA_ERR_NOMEM,
    FA_ERR_WORKSPACE,
    LIB_PATH,
    fa_bwd,
    fa_bwd_workspace_bytes,
    fa_decode,
    fa_decode_chunk_tokens,
    fa_decode_ex,
    fa_decode_fused,
    fa_decode_fused_workspace_bytes,
    fa_decode_noalloc,
    fa_decode_noalloc_scratch_bytes,
    fa_decode_paged,
    fa_decode_paged_splits,
    fa_decode_plan,
    fa_decode_workspace_bytes,
    fa_fwd,
    fa_fwd_f32,
    fa_fwd_plan,
    fa_get_fwd_exp2_poly,
    fa_set_fwd_exp2_poly,
    fa_probe_hbm_read,
    fa_probe_mfma_bf16,
    fa_probe_mfma_bf16_mixed,
    fa_release_workspace,
    last_error,
    lib,
    status_string,
)
