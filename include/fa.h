/*
 * fa.h -- exact attention forward (FlashAttention), its backward by
 * recomputation, and single-query Flash-Decoding for AMD MI355X (gfx950).
 * C ABI.
 *
 * Sources, cited by page title and section:
 *  [FA]  "Infra: Flash Attention" (pufanyi.com blog): "Attention and scope"
 *        (S = Q K^T / sqrt(d), row softmax, O = P V), "Tiled computation and
 *        forward" (Algorithm 1, FlashAttention forward; boundary conditions),
 *        "Backward and recomputation" (L_i = m_i + log l_i; recomputing P
 *        from L) and the tiled-gradient section after it, "Prefill and
 *        decode".
 *  [FD]  airsota interview card "Efficient attention & FlashAttention"
 *        (science-depth M4-055), section 3 "Mathematical principles &
 *        derivation": Flash-Decoding steps 1-3 (split the KV sequence into
 *        chunks, one partial (O^(k), m^(k), l^(k)) per chunk, log-sum-exp
 *        reduction), section 4 (choice of the chunk count).
 *  [L18] "CMU 10-423 Lecture 18" notes: section 3.4 (FA-2 loop order),
 *        section 4.3 (causal masks skip whole tiles), section 5.3 (the
 *        FlashAttention backward), section 7.3 (KV cache in blocks).
 *
 * Conventions shared by every entry point
 *  - Tensors are dense, row-major, with the head dimension d contiguous.
 *    Prefill tensors are [B, H, N, d]; L is [B, H, N].
 *  - Pointers documented as "device" must be device (or managed) memory on the
 *    current HIP device, 16-byte aligned.  The caller owns every buffer; the
 *    library neither frees nor retains caller pointers.  Outputs are fully
 *    overwritten and must not overlap any input.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued asynchronously on it; nothing here synchronises.
 *  - Return value: FA_OK (0) or a negative fa_status.  Arguments are validated
 *    on the host before any HIP call; an invalid call enqueues nothing.
 *    fa_last_error() then holds a message (thread-local).  Faults inside a
 *    kernel surface at the caller's next synchronisation, as for any HIP work.
 *  - Supported head dimensions: d = 64 and d = 128.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size or flag */
  FA_ERR_UNSUPPORTED = -2, /* valid request this build does not implement (e.g. d) */
  FA_ERR_HIP = -3,         /* a HIP runtime call or kernel launch failed */
  FA_ERR_NOMEM = -4,       /* the internal workspace could not be allocated */
  FA_ERR_WORKSPACE = -5    /* caller workspace missing or too small */
} fa_status;

/* Geometry of one fa_fwd launch (host-only planning; see fa_fwd_plan). */
typedef struct fa_fwd_plan_t {
  int block_rows;            /* B_r: query rows per workgroup */
  int block_cols;            /* B_c: keys per KV tile */
  int q_tiles;               /* ceil(N / B_r) per (b, h) */
  int kv_tiles;              /* ceil(N / B_c) per (b, h) */
  int threads_per_workgroup; /* wavefronts * 64 */
  int lds_bytes;             /* LDS per workgroup (d = 128: with output
                                staging rows) */
  int64_t workgroups;        /* causal or d = 128: min(work_units, compute
                                units); else work_units */
  int64_t tiles_visited;     /* (query tile, KV tile) pairs computed, all heads */
  int64_t tiles_masked;      /* of those, tiles masked on chip (diagonal/ragged) */
  int64_t work_units;        /* B * H * q_tiles, or B * H * ceil(q_tiles / 2)
                                causal pairs of query tiles (p, q_tiles-1-p) */
} fa_fwd_plan_t;

/* Geometry of one fa_decode launch (host-only planning; see fa_decode_plan). */
typedef struct fa_decode_plan_t {
  int num_splits;            /* chunks per (b, h) actually used */
  int threads_per_workgroup; /* split kernel */
  int64_t split_workgroups;  /* B * H * num_splits */
  int64_t combine_workgroups;/* B * H */
  size_t workspace_bytes;    /* partials: B*H*num_splits*(d + 1) floats, aligned */
} fa_decode_plan_t;

/*
 * fa_fwd -- FlashAttention forward, bf16 inputs ([FA] Algorithm 1, FA-2 order
 * per [L18] section 3.4).
 *   Q, K, V : device bf16 [B, H, N, d]
 *   O       : device bf16 [B, H, N, d], O = softmax(Q K^T * scale) V, each
 *             element rounded to nearest-even from fp32
 *   L       : device fp32 [B, H, N], natural-log log-sum-exp of the scaled
 *             scores of each row, L_i = m_i + log l_i; may be NULL (not written)
 *   causal  : 0 or 1; 1 keeps key j for query i iff j <= i (square, top-left
 *             aligned).  Tiles wholly above the diagonal are not visited
 *             ([L18] section 4.3).
 *   scale   : finite, > 0 (1/sqrt(d) for the pages' definition)
 * Arithmetic: bf16 MFMA products with fp32 accumulation; the softmax state
 * (m, l, U) is fp32; the probabilities fed to the second product are rounded
 * to bf16.  Errors: FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED (d), FA_ERR_HIP.
 */
int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* L, int B, int H,
           int N, int d, int causal, float scale, void* stream);

/*
 * fa_set_fwd_exp2_poly -- how many of the 64 exponentials per lane of a tile
 * the d = 128 bf16 forward evaluates by a polynomial on the multiply-add
 * units instead of the hardware exponential ([FA] "FlashAttention-4": part
 * of the exponentials on the FMA units, with the share to be chosen and
 * the approximation error to be evaluated).
 *   per64 : 0 (the default: hardware exponential only), 4, 8 or 16.  The
 *           polynomial is a cubic in the fraction of the exponent, maximum
 *           relative error 8.6e-5 (below the bf16 rounding of the
 *           probabilities), scaled by the integer part through the exponent.
 * Process-wide; read by each later fa_fwd call (calls already enqueued keep
 * their setting).  d = 64 and fa_fwd_f32 are not affected.
 * Errors: FA_ERR_INVALID_ARG for any other value (the setting is unchanged).
 * fa_get_fwd_exp2_poly returns the current setting.
 */
int fa_set_fwd_exp2_poly(int per64);
int fa_get_fwd_exp2_poly(void);

/*
 * fa_fwd_f32 -- the same contract with fp32 Q, K, V, O (device fp32
 * [B, H, N, d]); every operation is fp32 (no reduced-precision step).
 */
int fa_fwd_f32(const float* Q, const float* K, const float* V, float* O, float* L, int B,
               int H, int N, int d, int causal, float scale, void* stream);

/*
 * fa_bwd -- gradients of the FlashAttention forward by recomputation ([FA]
 * "Backward and recomputation" and its tiled-gradient section; [L18]
 * section 5.3).
 *   Q, K, V : device bf16 [B, H, N, d], the forward's inputs
 *   O, L    : the forward's outputs (bf16 [B, H, N, d] and fp32 [B, H, N],
 *             natural-log log-sum-exp of the scaled scores) for the same Q,
 *             K, V, causal and scale
 *   dO      : device bf16 [B, H, N, d], the gradient of the loss w.r.t. O
 *   dQ, dK, dV : device bf16 [B, H, N, d], fully overwritten:
 *             D_i = dO_i . O_i, P_ij = exp(S_ij - L_i) with S = Q K^T scale
 *             (causal: P_ij = 0 for j > i), dV = P^T dO, dS = P o (dO V^T -
 *             D), dQ = scale dS K, dK = scale dS^T Q; each element rounded to
 *             nearest-even from fp32
 *   causal, scale : as in fa_fwd
 *   workspace : device memory of at least fa_bwd_workspace_bytes(B, H, N)
 *             bytes, 256-byte aligned, for D and L log2 e; or NULL with workspace_bytes = 0
 *             to use the library's workspace of the (device, stream) (grown
 *             with hipMalloc, so not while the stream is being captured)
 * Arithmetic: bf16 MFMA products with fp32 accumulation; P and dS are rounded
 * to bf16 as product operands; D, P, dP and dS are computed in fp32.  The
 * result does not depend on timing (no atomics).  The inputs may overlap
 * each other; the outputs may not overlap an input, L, the workspace or each
 * other.  Errors: FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED (d), FA_ERR_WORKSPACE,
 * FA_ERR_NOMEM, FA_ERR_HIP.
 */
int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* L,
           void* dQ, void* dK, void* dV, int B, int H, int N, int d, int causal, float scale,
           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes fa_bwd needs (two arrays of B * H * N floats, each
 * rounded up to 256 bytes); 0 for invalid arguments. */
size_t fa_bwd_workspace_bytes(int B, int H, int N);

/*
 * fa_decode -- Flash-Decoding of one query per (b, h) against a KV cache
 * ([FA] "Prefill and decode"; [FD] section 3 steps 1-3).
 *   q       : device bf16 [B, H, d] (the newest token's query)
 *   Kcache, Vcache : device bf16, packed by sequence: sequence b occupies a
 *             [H, Lkv[b], d] block and the blocks follow each other in b
 *             order (so equal lengths give plain [B, H, L, d])
 *   o       : device bf16 [B, H, d]
 *   Lkv     : device int32 [B], per-sequence cache lengths (>= 0).  A length
 *             of 0 gives o = 0 for that sequence.
 *   num_splits : chunks per (b, h); 0 = automatic: ceil(CUs / (B * H))
 *             clamped to [8, 256], CUs being the device's compute units.  Sequence b is cut into chunks of
 *             ceil(Lkv[b] / num_splits) tokens rounded up to a multiple of 64;
 *             trailing chunks may be empty.
 * The query attends to every cached key with scale 1/sqrt(d).  Partials go to
 * an internal workspace owned by the library, one per (device, stream), grown
 * on demand with hipMalloc (so not while the stream is being captured) and
 * released by fa_release_workspace().  Errors: FA_ERR_INVALID_ARG,
 * FA_ERR_UNSUPPORTED, FA_ERR_NOMEM, FA_ERR_HIP.
 */
int fa_decode(const void* q, const void* Kcache, const void* Vcache, void* o, int B, int H,
              const int32_t* Lkv, int d, int num_splits, void* stream);

/*
 * fa_decode_ex -- fa_decode with every option explicit.
 *   lse_out         : device fp32 [B, H] or NULL; natural-log log-sum-exp of
 *                     the query's scaled scores (-inf for an empty cache)
 *   kv_seq_capacity : 0 = packed layout as in fa_decode; > 0 = padded layout
 *                     [B, H, kv_seq_capacity, d] with Lkv[b] <= capacity
 *                     (lengths above it are clamped to it)
 *   scale           : finite, > 0
 *   workspace       : caller-owned device memory of at least
 *                     fa_decode_workspace_bytes(B, H, d, num_splits) bytes,
 *                     256-byte aligned; it must not be shared by calls that
 *                     may run concurrently.
 * Allocates nothing.  Errors: as fa_decode, plus FA_ERR_WORKSPACE.
 */
int fa_decode_ex(const void* q, const void* Kcache, const void* Vcache, void* o,
                 float* lse_out, int B, int H, const int32_t* Lkv, int kv_seq_capacity, int d,
                 int num_splits, float scale, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * fa_decode_fused -- fa_decode_ex in one launch: the last split workgroup of
 * each (b, h) to finish performs the log-sum-exp merge (the airsota
 * Flash-Decoding card, section 3, steps 1-3, with step 3 moved into the
 * kernel of steps 1-2; "Infra: Flash Attention", "Prefill and decode": the
 * merge order is free).
 *   q, Kcache, Vcache, o, lse_out, Lkv, kv_seq_capacity, num_splits, scale :
 *             as in fa_decode_ex
 *   B * H   : at most 65536 (FA_ERR_UNSUPPORTED above)
 *   workspace : caller-owned device memory of at least
 *             fa_decode_fused_workspace_bytes(B, H, d, num_splits) bytes,
 *             256-byte aligned: 65536 int32 counters (256 KiB), then the
 *             split partials.  The counters must be zero before the first
 *             call (for example a zero-filled allocation); each call that
 *             completes leaves them zero again, so the workspace can be
 *             reused call after call, for any shape that fits it.  Calls
 *             that may run concurrently must not share one.
 * Results are bit-identical to fa_decode_ex with the same arguments.
 * Publishing a partial to a workgroup that may run on another XCD needs an
 * agent-scope release per split workgroup, which on MI355X costs more than
 * the second launch it saves: fa_decode_ex is the faster path.
 * Allocates nothing.  Errors: as fa_decode_ex.
 */
int fa_decode_fused(const void* q, const void* Kcache, const void* Vcache, void* o, float* lse_out,
                    int B, int H, const int32_t* Lkv, int kv_seq_capacity, int d, int num_splits,
                    float scale, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes fa_decode_fused needs (0 for invalid arguments). */
size_t fa_decode_fused_workspace_bytes(int B, int H, int d, int num_splits);

/*
 * fa_decode_noalloc -- fa_decode_ex without a workspace argument and without
 * any allocation, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *   q, Kcache, Vcache, o, lse_out, Lkv, kv_seq_capacity, num_splits, scale :
 *             as in fa_decode_ex
 * The split partials go to a static device array inside the library, one per
 * device, of fa_decode_noalloc_scratch_bytes() bytes (4 MiB: for example
 * B * H * num_splits up to 8128 partials at d = 128), held until the process
 * ends.  A request whose partials (fa_decode_workspace_bytes) exceed it is
 * rejected with FA_ERR_WORKSPACE before anything is enqueued.  Every call on
 * a device shares that device's array: calls that may overlap on one device
 * (concurrent streams, other host threads) race and must be ordered by the
 * caller.  Results are identical to fa_decode_ex with the same arguments.
 * Errors: as fa_decode_ex.
 */
int fa_decode_noalloc(const void* q, const void* Kcache, const void* Vcache, void* o, float* lse_out,
                      int B, int H, const int32_t* Lkv, int kv_seq_capacity, int d, int num_splits,
                      float scale, void* stream);

/* Size in bytes of fa_decode_noalloc's per-device scratch. */
size_t fa_decode_noalloc_scratch_bytes(void);

/* Workspace bytes fa_decode_ex needs; num_splits = 0 resolves the automatic
 * count on the current device.  Returns 0 for invalid arguments. */
size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits);

/*
 * fa_decode_paged -- Flash-Decoding against a KV cache kept in fixed-size
 * blocks and read through a block table ([L18] section 7.3: blocks of a fixed
 * number of tokens, a table from each sequence's logical blocks to physical
 * ones, attention computed block by block and merged with the (m, l, o) state
 * of section 2.3).
 *   q, o, lse_out, Lkv, scale : as in fa_decode_ex
 *   Kpool, Vpool : device bf16 [num_blocks, H, block_size, d]; physical
 *             block p holds block_size consecutive tokens of every head
 *   block_table : device int32 [B, max_blocks], row-major; entry [b, i] is
 *             the physical block of tokens i*block_size .. (i+1)*block_size-1
 *             of sequence b.  Only entries i < ceil(Lkv[b] / block_size) are
 *             read.  An entry outside [0, num_blocks) is never dereferenced:
 *             its tokens are skipped (they contribute nothing).
 *   Lkv     : device int32 [B]; lengths above max_blocks * block_size are
 *             clamped to it
 *   block_size : a power of two in [16, 65536]
 *   num_splits : chunks per (b, h), 0 = automatic (fa_decode's rule, raised
 *             until no chunk spans more than 2048 blocks); an explicit count
 *             that lets a chunk span more is rejected (FA_ERR_UNSUPPORTED).
 *   workspace : caller-owned device memory of at least
 *             fa_decode_workspace_bytes(B, H, d, S) bytes for the split count
 *             S that fa_decode_paged_splits reports, 256-byte aligned; or NULL
 *             with workspace_bytes = 0 to use the library's workspace (as
 *             fa_decode: grown with hipMalloc outside stream capture only).
 * Identical keys give results identical to fa_decode_ex on a contiguous
 * cache with the same split count.  Errors: as fa_decode_ex.
 */
int fa_decode_paged(const void* q, const void* Kpool, const void* Vpool, void* o, float* lse_out,
                    int B, int H, const int32_t* block_table, int max_blocks, const int32_t* Lkv,
                    int num_blocks, int block_size, int d, int num_splits, float scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/* The split count fa_decode_paged uses for these arguments (resolving
 * num_splits = 0 on the current device, or for 256 compute units without
 * one); 0 if the arguments are invalid or no count keeps every chunk within
 * 2048 blocks. */
int fa_decode_paged_splits(int B, int H, int max_blocks, int block_size, int num_splits);

/* Host-only launch planning (no HIP call; usable without a GPU).
 * fa_fwd_plan: tile geometry and the exact number of tiles fa_fwd visits.
 * Causal fa_fwd runs a persistent grid of one workgroup per compute unit,
 * each taking every grid-th pair of query tiles; so does non-causal fa_fwd
 * at d = 128, with single query tiles.  Without a device the plan assumes
 * 256 compute units.  Non-causal fa_fwd at d = 64 runs one workgroup per
 * query tile.
 * fa_decode_plan: splits and workspace; num_splits = 0 needs the device's CU
 * count, so without a device it assumes 256 compute units.
 * fa_decode_chunk_tokens: chunk length for a sequence of kv_len tokens. */
int fa_fwd_plan(int B, int H, int N, int d, int causal, fa_fwd_plan_t* out);
int fa_decode_plan(int B, int H, int d, int num_splits, fa_decode_plan_t* out);
int fa_decode_chunk_tokens(int kv_len, int num_splits);

/* Frees the internal workspaces of fa_decode, fa_decode_paged and fa_bwd
 * (synchronises the devices that own them).  Returns FA_OK or FA_ERR_HIP. */
int fa_release_workspace(void);

/* Measurement kernels (no attention): the measured ceilings that a roofline
 * places next to the published peaks ("CMU 10-423 Lecture 18", section 6,
 * the roofline model).
 *
 * fa_probe_hbm_read: reads every 16-byte word of buf once (workgroups of 256
 * threads striding over the buffer, eight loads in flight per thread) and
 * writes nothing but, with negligible probability, one word of sink.
 *   buf   : device, 16-byte aligned, `bytes` readable bytes
 *   bytes : > 0, a multiple of 16
 *   workgroups : in [1, 1048576]
 *   sink  : device uint32 [workgroups], 4-byte aligned, not overlapping buf
 * Algorithmic traffic: `bytes` read per launch.
 *
 * fa_probe_mfma_bf16: every wavefront of `workgroups` x 4 runs `iters` rounds
 * of four independent v_mfma_f32_32x32x16_bf16 (32768 FLOP each), i.e.
 * workgroups * 4 * iters * 4 * 32768 FLOP per launch.
 *   workgroups : in [1, 1048576]; iters : in [1, 16777216]
 *   sink  : device float [workgroups * 256], 4-byte aligned (one value per
 *           thread, so the products cannot be dropped)
 *   stamps: device uint64 [2 * workgroups], 8-byte aligned, or NULL; for
 *           each workgroup, the shader-clock cycles and the 100 MHz
 *           constant-clock ticks its first wavefront spent in the loop
 *           (cycles / (ticks / 1e8) = the clock it ran at)
 *
 * fa_probe_mfma_bf16_mixed: the same loop and arguments, but every chain has
 * its own A and B operands, pseudo-random in [-2, 2) (an integer hash of
 * seed, workgroup, lane, chain and element), so consecutive products read
 * different data, as the attention kernels' products do.  The constant loop
 * multiplies small multiples of 0.001 and 0.002, many of them zero; with
 * random bf16 values held constant it runs within 4 % of this loop: the
 * operand values, more than their changing between products, set the power
 * the products draw and so the clock.
 * All three: errors FA_ERR_INVALID_ARG (checked before any HIP call),
 * FA_ERR_HIP. */
int fa_probe_hbm_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink, void* stream);
int fa_probe_mfma_bf16(int workgroups, int iters, float* sink, uint64_t* stamps, void* stream);
int fa_probe_mfma_bf16_mixed(int workgroups, int iters, uint32_t seed, float* sink, uint64_t* stamps,
                             void* stream);

/* Static description of a status code, and the thread-local message of the
 * last failing call on this thread ("" if none). */
const char* fa_status_string(int status);
const char* fa_last_error(void);

/* Library ABI version: (major << 16) | minor. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
