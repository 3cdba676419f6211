// Internal declarations shared by the host dispatch (fa_api.hip) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Prefill tiling, shared by the planner and the bf16 kernel: a workgroup of
// kFwdWaves wavefronts owns kFwdBR query rows (32 per wavefront) and walks
// KV tiles of kFwdBC keys.
constexpr int kFwdWaves = 8;
constexpr int kFwdBR = 32 * kFwdWaves;
// B_c is fixed at 64.  The buffer->LDS load helper pads its asm with
// wait states for the SGPR operands it reads (fa_device.h, load_lds16); that
// padding has been exercised with these tiles only, so no other B_c is
// built.
constexpr int kFwdBC = 64;
// LDS of one prefill workgroup: two K and two V tiles, each row padded by 16
// bytes (the query tile lives in registers).
__host__ __device__ constexpr int fwd_lds_bytes(int d) { return 4 * kFwdBC * (2 * d + 16); }
// LDS of the d = 128 kernel with generated assembly: the same K/V buffers
// plus 256 padded output staging rows.
__host__ __device__ constexpr int fwd_asm_lds_bytes() { return fwd_lds_bytes(128) + 256 * (2 * 128 + 16); }

// fp32 prefill: one wavefront, one query row per lane, 64-key tiles.
constexpr int kF32BR = 64;
constexpr int kF32BC = 64;

// bf16 backward: wavefronts per workgroup (two workgroups per compute unit,
// so two wavefronts per SIMD); the dK/dV kernel
// gives each wavefront 32 keys (kBwdKV per workgroup) and walks query tiles
// of kBwdQT rows; the dQ kernel gives each wavefront 32 queries (kBwdQ per
// workgroup) and walks KV tiles of kBwdKT keys.  LDS: two buffers of
// (Q tile, dO tile, 1 KiB of L, 1 KiB of D), resp. (K tile, V tile), rows
// padded by 16 bytes.
constexpr int kBwdWaves = 4;
constexpr int kBwdKV = 32 * kBwdWaves;
constexpr int kBwdQT = 32;
constexpr int kBwdQ = 32 * kBwdWaves;
constexpr int kBwdKT = 64;
__host__ __device__ constexpr int bwd_tile_bytes(int rows, int d) { return (rows * (2 * d + 16) + 1023) / 1024 * 1024; }
__host__ __device__ constexpr int bwd_dkdv_lds_bytes(int d) { return 2 * (2 * bwd_tile_bytes(kBwdQT, d) + 2 * 1024); }
__host__ __device__ constexpr int bwd_dq_lds_bytes(int d) { return 2 * 2 * bwd_tile_bytes(kBwdKT, d); }

// Decode split kernel: wavefronts per workgroup; chunk lengths are rounded up
// to a multiple of kDecChunkAlign tokens.
constexpr int kDecWaves = 4;
constexpr int kDecChunkAlign = 64;
// Paged decode: block ids one split workgroup stages in LDS (the host picks
// split counts so that no chunk spans more blocks), and the block sizes
// accepted (powers of two).
constexpr int kPagedIdsPerChunk = 2048;
constexpr int kPagedMinBlock = 16;
constexpr int kPagedMaxBlock = 65536;

struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* L;
  int B, H, N;
  int causal;
  float scale;
  int grid;  // bf16 prefill: persistent workgroups, 1 <= grid <= fwd_units
  int exp2_poly = 0;  // d = 128 bf16: exponentials per 64 by polynomial (0, 4, 8, 16)
};

struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* L;
  void* dQ;
  void* dK;
  void* dV;
  float* Dws;   // [B, H, N] fp32 workspace: D_i = dO_i . O_i
  float* L2ws;  // [B, H, N] fp32 workspace: L_i log2 e
  int B, H, N;
  int causal;
  float scale;
};

struct DecodeArgs {
  const void* q;
  const void* K;
  const void* V;
  void* o;
  float* lse_out;
  const int32_t* Lkv;
  float* part_o;    // [B, H, S, d]
  float* part_lse;  // [B, H, S]
  int B, H, S;
  int capacity;     // 0 = packed
  float scale;
  // paged cache (table != nullptr): K/V are pools [num_blocks, H, 2^log2_bs, d]
  const int32_t* table = nullptr;  // [B, max_blocks]
  int max_blocks = 0, log2_bs = 0, num_blocks = 0;
  // one launch: per-(b, h) counters [B, H], zero on entry and on exit
  int* counters = nullptr;
};

// bf16 prefill with d = 128 runs the 64-rows-per-wavefront kernel (4
// wavefronts of 64 query rows, tile loop in generated assembly); d = 64 the
// 32-rows-per-wavefront one (8 wavefronts).  Both use the tiles above.
inline bool fwd_uses_asm(int d, int causal) { (void)causal; return d == 128; }
inline int fwd_lds_for(int d, int causal) { return fwd_uses_asm(d, causal) ? fwd_asm_lds_bytes() : fwd_lds_bytes(d); }
inline int fwd_threads(int d, int causal) { return fwd_uses_asm(d, causal) ? 4 * 64 : kFwdWaves * 64; }

// Launchers: enqueue on `stream`, return hipGetLastError().
hipError_t launch_fwd_bf16(const FwdArgs& a, int d, hipStream_t stream);
hipError_t launch_fwd_bf16_asm(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, int d, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int d, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs& a, int d, hipStream_t stream);
hipError_t launch_probe_hbm_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink,
                                 hipStream_t stream);
hipError_t launch_probe_mfma_bf16(int workgroups, int iters, float* sink, uint64_t* stamps, hipStream_t stream);
hipError_t launch_probe_mfma_bf16_mixed(int workgroups, int iters, uint32_t seed, float* sink, uint64_t* stamps,
                                        hipStream_t stream);

// Host-side tile bookkeeping used by both the planner and the launcher.
__host__ __device__ inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Number of KV tiles that query tile `qt` visits (causal tiles wholly in the
// future are skipped).
inline int fwd_kv_tiles_for(int qt, int N, int causal) {
  int kv_tiles = (int)ceil_div64(N, kFwdBC);
  if (!causal) return kv_tiles;
  int last_row = (qt + 1) * kFwdBR - 1;
  if (last_row > N - 1) last_row = N - 1;
  int t = last_row / kFwdBC + 1;
  return t < kv_tiles ? t : kv_tiles;
}

// Work units of the persistent bf16 prefill grid: one query tile, or for
// causal attention the pair of query tiles (p, q_tiles-1-p) of a head.
inline int64_t fwd_units(int B, int H, int N, int causal) {
  const int64_t q_tiles = ceil_div64(N, kFwdBR);
  return (int64_t)B * H * (causal ? (q_tiles + 1) / 2 : q_tiles);
}
// Grid of the bf16 prefill.  Persistent, one workgroup per compute unit
// (fewer if there are fewer units), each taking every grid-th unit: always
// for causal attention (pairs of query tiles, so all workgroups get the same
// work) and for the kernel with generated assembly (whose items prefetch
// their successor's loads).  Otherwise one workgroup per unit, which lets the
// hardware overlap one workgroup's start with another's end.
inline int64_t fwd_grid(int64_t units, int d, int causal, int cus) {
  const bool persistent = causal || fwd_uses_asm(d, causal);
  return persistent ? (units < cus ? units : cus) : units;
}

// Blocks a chunk of at most chunk_tokens tokens can touch when chunks start
// at multiples of kDecChunkAlign and blocks hold block_size tokens.
inline int64_t paged_blocks_per_chunk(int64_t chunk_tokens, int block_size) {
  return ceil_div64(chunk_tokens, block_size) + 1;
}

// Decode chunk length for a sequence of `len` tokens split `S` ways.
__host__ __device__ inline int decode_chunk_tokens(int len, int S) {
  if (len <= 0 || S <= 0) return 0;
  int64_t c = ceil_div64(len, S);
  c = ceil_div64(c, kDecChunkAlign) * kDecChunkAlign;
  return (int)c;
}

}  // namespace fa
