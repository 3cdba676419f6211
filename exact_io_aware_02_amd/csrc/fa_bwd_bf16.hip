// FlashAttention backward for bf16 Q/K/V on gfx950 (MI355X).
//
// What it computes ("Infra: Flash Attention", sections "Backward and
// recomputation" and the tiled-gradient section after it; "CMU 10-423
// Lecture 18" notes, section 5.3): given the forward's O and per-row
// log-sum-exp L, and the upstream gradient G = dO,
//     D_i  = G_i . O_i
//     P_ij = exp(S_ij - L_i),   S = Q K^T * scale (causal: 0 for j > i)
//     dV = P^T G,   dP = G V^T,   dS = P o (dP - D)
//     dQ = scale dS K,   dK = scale dS^T Q
// with P, dP and dS recomputed tile by tile and never stored.
//
// Three launches, no atomics (so results do not depend on timing):
//  1. bwd_dot_kernel: D for every row, and L in base 2 (L log2 e) so that
//     P = exp2(S scale log2 e - L log2 e) is one fma and one exp2 per element
//     (HBM-bound, 2 N d bf16 reads per head).
//  2. bwd_dkdv_kernel: a workgroup owns kBwdKV keys (32 per wavefront, K and
//     V held in registers as MFMA B operands) and walks query tiles of
//     kBwdQT rows staged in LDS with their L and D: S, P, dV^T += dO^T P,
//     dP, dS, dK^T += Q^T dS.  Four products per tile (8 N^2 d flops per
//     head).
//  3. bwd_dq_kernel: a workgroup owns kBwdQ queries (32 per wavefront, Q and
//     dO in registers) and walks KV tiles of kBwdKT keys: S^T = K Q^T,
//     dP^T = V dO^T, dS^T, dQ^T += K^T dS^T (6 N^2 d flops per head): the
//     forward's structure, with P exact from L instead of an online max.
// The dQ reduction over key tiles therefore runs inside one workgroup, at
// the price of recomputing S and dP once more (14 instead of 10 N^2 d flops
// per head); accumulating dQ across workgroups with atomics would put
// (N / kBwdKV) N d fp32 read-modify-writes per head through the L2.
//
// Occupancy: both kernels fit 256 registers per lane, so two workgroups of
// four wavefronts share a compute unit and each SIMD interleaves two
// wavefronts' matrix, exponential and LDS work (measured on prefill_8k: 3.97
// ms against 6.27 ms with one wavefront per SIMD and 64-row query tiles).
//
// CDNA4 mapping, shared with the forward (fa_device.h):
//  * v_mfma_f32_32x32x16_bf16 throughout; accumulators hold 32 x 32 blocks
//    with the column on the lane, so row statistics (L, D) are per register
//    in the KV-outer kernel and per lane in the Q-outer one;
//  * tiles go HBM -> LDS with buffer->LDS loads (rows past N read as zeros),
//    rows padded by 16 bytes and stored with vrow_perm, so the 16-byte row
//    fragment reads (natural row order through a per-lane permuted base) and
//    the transposing reads (ds_read_b64_tr_b16) of the same tile are both
//    conflict-free;
//  * probabilities and score gradients leave their fp32 accumulators already
//    in the B-operand layout of the next product (bf16), as W does in the
//    forward; exponentials run in base 2 with scale*log2(e) folded in.

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

using namespace dev;

constexpr int kThreads = kBwdWaves * 64;

template <int D>
struct BwdTile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kStride = kRowBytes + 16;  // padded LDS row
  // LDS regions are whole KiB (the loads move 1 KiB per wavefront
  // instruction); slack after a tile's rows receives the following rows, or
  // zeros past N, and is never read
  static constexpr int kQTBytes = bwd_tile_bytes(kBwdQT, D);  // a query (or dO) tile of the KV-outer kernel
  static constexpr int kKTBytes = bwd_tile_bytes(kBwdKT, D);  // a K (or V) tile of the Q-outer kernel
  static constexpr int kStatBytes = 1024;                     // L or D of one query tile (zero-padded)
  static constexpr int kDkdvLds = 2 * (2 * kQTBytes + 2 * kStatBytes);
  static constexpr int kDqLds = 2 * 2 * kKTBytes;
  static_assert(kDkdvLds == bwd_dkdv_lds_bytes(D) && kDqLds == bwd_dq_lds_bytes(D), "LDS size must match the planner");
};

// A bf16x8 from 8 floats (round to nearest even).
__device__ __forceinline__ bf16x8_t to_bf16x8(const float* p) {
  return bf16x8_t{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                  (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
}

// Copies `bytes` (a multiple of 1 KiB) of padded rows into LDS: every
// wavefront of the workgroup issues its share of 1 KiB loads.  `voff_of`
// gives the per-lane source offset of LDS byte o within the tile, `soff` the
// tile's offset in the head (the SGPR offset, which gfx950 includes in the
// range check: rows past the head read zeros).
template <typename F>
__device__ __forceinline__ void dma_rows(const u32x4_t rsrc, unsigned soff, char LDS_AS* dst, int bytes, int wave,
                                         int lane, F voff_of) {
  for (int blk = wave; blk < bytes / 1024; blk += kBwdWaves)
    load_lds16(rsrc, (void LDS_AS*)(dst + blk * 1024), voff_of(blk * 1024 + lane * 16), soff);
}

// Output rows of 32 x D in the accumulator layout (lane = row, registers =
// columns 32 db + 8 i4 + 4 g + 0..3), times `mul`, as bf16.
template <int D>
__device__ __forceinline__ void store_rows(__bf16* base, int row, int N, const f32x16_t (&acc)[D / 32], float mul,
                                           int g) {
  if (row >= N) return;
  __bf16* r = base + (size_t)row * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      u32x2_t v;
      v[0] = pack_bf16x2(acc[db][4 * i4 + 0] * mul, acc[db][4 * i4 + 1] * mul);
      v[1] = pack_bf16x2(acc[db][4 * i4 + 2] * mul, acc[db][4 * i4 + 3] * mul);
      *reinterpret_cast<u32x2_t*>(r + db * 32 + 8 * i4 + 4 * g) = v;
    }
  }
}

// Logical index of workgroup b of G such that the workgroups placed on one
// XCD (the dispatcher deals workgroups round-robin over the 8 XCDs) get
// consecutive logical indices, so one head's items run on one XCD and share
// its L2.  A bijection on [0, G) whatever the actual placement.
__device__ __forceinline__ int xcd_local_index(int b, int G) {
  const int per = G >> 3, rem = G & 7;
  const int xcd = b & 7, slot = b >> 3;
  return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

// ---------------------------------------------------------------------------
// 1. D_i = G_i . O_i
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_dot_kernel(const __bf16* __restrict__ O, const __bf16* __restrict__ dO,
                                                      const float* __restrict__ L, float* __restrict__ Dout,
                                                      float* __restrict__ L2out, long long rows) {
  constexpr int LPR = D / 8;       // lanes per row (16 bytes each)
  constexpr int RPW = 64 / LPR;    // rows per wavefront
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long row = ((long long)blockIdx.x * 4 + wave) * RPW + lane / LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(O + row * D + (lane % LPR) * 8);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(dO + row * D + (lane % LPR) * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = __builtin_fmaf(__uint_as_float(a[w] << 16), __uint_as_float(b[w] << 16), acc);
      acc = __builtin_fmaf(__uint_as_float(a[w] & 0xffff0000u), __uint_as_float(b[w] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off);
  if (row < rows && lane % LPR == 0) {
    Dout[row] = acc;
    L2out[row] = L[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// 2. dK, dV: one workgroup per kBwdKV keys of one head
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(const __bf16* __restrict__ Qg, const __bf16* __restrict__ Kg, const __bf16* __restrict__ Vg,
                     const __bf16* __restrict__ dOg, const float* __restrict__ L2g, const float* __restrict__ Dg,
                     __bf16* __restrict__ dKg, __bf16* __restrict__ dVg, int N, int kv_tiles, float scale) {
  using T = BwdTile<D>;
  // per buffer s: [Q tile][dO tile][L][D]
  __shared__ __attribute__((aligned(1024))) char smem[T::kDkdvLds];
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  char LDS_AS* lds = (char LDS_AS*)smem;
  constexpr int kBuf = 2 * T::kQTBytes + 2 * T::kStatBytes;
  auto qbuf = [&](int s) { return lds + s * kBuf; };
  auto dobuf = [&](int s) { return lds + s * kBuf + T::kQTBytes; };
  auto lbuf = [&](int s) { return (const float LDS_AS*)(lds + s * kBuf + 2 * T::kQTBytes); };
  auto dbuf = [&](int s) { return (const float LDS_AS*)(lds + s * kBuf + 2 * T::kQTBytes + T::kStatBytes); };

  // work item: key tile kt of head bh, head-major over XCD-local logical
  // indices (a head's Q and dO tiles are re-read by all its key tiles, from
  // one L2); within a head the longest causal items (first key tiles) first
  const int lw = xcd_local_index(blockIdx.x, gridDim.x);
  const int bh = lw / kv_tiles;
  const int kt = lw - bh * kv_tiles;
  const size_t head = (size_t)bh * N * D;
  const unsigned head_bytes = (unsigned)N * D * 2;
  const int key = kt * kBwdKV + wave * 32 + l32;  // this lane's key (column of every accumulator)

  // K and V rows of the lane's key as B operands: lane (l32, g) holds
  // elements 16 ds + 8 g + 0..7
  bf16x8_t kf[D / 16], vf[D / 16];
  {
    const bf16x8_t* kp = reinterpret_cast<const bf16x8_t*>(Kg + head + (size_t)key * D) + g;
    const bf16x8_t* vp = reinterpret_cast<const bf16x8_t*>(Vg + head + (size_t)key * D) + g;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      kf[ds] = key < N ? kp[2 * ds] : bf16x8_t{};
      vf[ds] = key < N ? vp[2 * ds] : bf16x8_t{};
    }
  }
  f32x16_t dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dk[db] = dv[db] = f32x16_t{};

  // query tiles: causal items skip tiles whose every query precedes every key
  const int n_qt = (N + kBwdQT - 1) / kBwdQT;
  const int qt0 = CAUSAL ? (kt * kBwdKV) / kBwdQT : 0;
  const u32x4_t q_rsrc = make_rsrc(Qg + head, head_bytes);
  const u32x4_t do_rsrc = make_rsrc(dOg + head, head_bytes);
  const u32x4_t l_rsrc = make_rsrc(L2g + (size_t)bh * N, (unsigned)N * 4);
  const u32x4_t d_rsrc = make_rsrc(Dg + (size_t)bh * N, (unsigned)N * 4);
  auto issue = [&](int t, int s) {
    const unsigned soff = (unsigned)t * kBwdQT * T::kRowBytes;
    dma_rows(q_rsrc, soff, qbuf(s), T::kQTBytes, wave, lane, [](int o) { return padded_source<D>(o, true); });
    dma_rows(do_rsrc, soff, dobuf(s), T::kQTBytes, wave, lane, [](int o) { return padded_source<D>(o, true); });
    // 64 floats of L and D (lanes past them read zeros into the padding)
    if (wave == 0) {
      const unsigned so = (unsigned)t * kBwdQT * 4;
      const unsigned vo = lane < kBwdQT / 4 ? (unsigned)lane * 16 : 0x7FFFFFF0u;
      load_lds16(l_rsrc, (void LDS_AS*)lbuf(s), vo, so);
      load_lds16(d_rsrc, (void LDS_AS*)dbuf(s), vo, so);
    }
  };

  const float c = scale * kLog2e;
  // per-lane LDS bases: 16-byte fragments of natural row l32 (stored at
  // vrow_perm(l32)), and the transposing-read base
  const int row_base = vrow_perm(l32) * T::kStride + g * 16;
  const int tr_base = tr_lane_base<T::kStride>(lane);

  if (qt0 < n_qt) issue(qt0, 0);
  for (int t = qt0; t < n_qt; ++t) {
    const int s = (t - qt0) & 1;
    wait_vmem();
    wg_barrier();  // every wavefront's share of tile t has landed; tile t-1 is no longer read
    if (t + 1 < n_qt) issue(t + 1, s ^ 1);
    const char LDS_AS* qtile = qbuf(s);
    const char LDS_AS* otile = dobuf(s);
    const int q0 = t * kBwdQT;
    // every (query, key) pair of this wavefront's tile is valid: no per-element
    // masks (all tiles but a ragged last one and, causal, the diagonal ones)
    const bool full = q0 + kBwdQT <= N && (!CAUSAL || kt * kBwdKV + wave * 32 + 31 <= q0);

    // S = Q K^T (query rows, the lane's key in the column), 2 blocks of 32 queries
    f32x16_t sc[kBwdQT / 32], dp[kBwdQT / 32];
#pragma unroll
    for (int qb = 0; qb < kBwdQT / 32; ++qb) sc[qb] = dp[qb] = f32x16_t{};
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
#pragma unroll
      for (int qb = 0; qb < kBwdQT / 32; ++qb) {
        const bf16x8_t a = *(const bf16x8_t LDS_AS*)(qtile + row_base + qb * 32 * T::kStride + ds * 32);
        sc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[ds], sc[qb], 0, 0, 0);
      }
    }
    // P = exp2(S c - L_row log2 e) (L staged in base 2); rows past N and
    // (causal) queries before the key get 0.  Element i of block qb is query
    // q0 + 32 qb + 8 (i >> 2) + 4 g + (i & 3).
    bf16x8_t pb[kBwdQT / 16];
    float pf[kBwdQT / 32][16];
    if (full) {
#pragma unroll
      for (int qb = 0; qb < kBwdQT / 32; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f32x4_t L4 = *(const f32x4_t LDS_AS*)(lbuf(s) + 32 * qb + 8 * r + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pf[qb][4 * r + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qb][4 * r + e], c, -L4[e]));
        }
    } else {
#pragma unroll
      for (int qb = 0; qb < kBwdQT / 32; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rl = 32 * qb + 8 * r + 4 * g;  // first of 4 consecutive local rows
          const f32x4_t L4 = *(const f32x4_t LDS_AS*)(lbuf(s) + rl);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int qrow = q0 + rl + e;
            const bool ok = qrow < N && (!CAUSAL || key <= qrow);
            pf[qb][4 * r + e] = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qb][4 * r + e], c, -L4[e])) : 0.f;
          }
        }
    }
#pragma unroll
    for (int qb = 0; qb < kBwdQT / 32; ++qb)
#pragma unroll
      for (int h = 0; h < 2; ++h) pb[2 * qb + h] = to_bf16x8(&pf[qb][8 * h]);
    // dV^T += dO^T P (queries are the contraction index)
#pragma unroll
    for (int ks = 0; ks < kBwdQT / 16; ++ks) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8_t a = tr_frag<T::kStride>(otile + tr_base, ks, db * 64);
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks], dv[db], 0, 0, 0);
      }
    }
    // dP = dO V^T
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
#pragma unroll
      for (int qb = 0; qb < kBwdQT / 32; ++qb) {
        const bf16x8_t a = *(const bf16x8_t LDS_AS*)(otile + row_base + qb * 32 * T::kStride + ds * 32);
        dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[ds], dp[qb], 0, 0, 0);
      }
    }
    // dS = P (dP - D_row)
    bf16x8_t dsb[kBwdQT / 16];
#pragma unroll
    for (int qb = 0; qb < kBwdQT / 32; ++qb) {
      float dsf[16];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4_t D4 = *(const f32x4_t LDS_AS*)(dbuf(s) + 32 * qb + 8 * r + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) dsf[4 * r + e] = pf[qb][4 * r + e] * (dp[qb][4 * r + e] - D4[e]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) dsb[2 * qb + h] = to_bf16x8(&dsf[8 * h]);
    }
    // dK^T += Q^T dS
#pragma unroll
    for (int ks = 0; ks < kBwdQT / 16; ++ks) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8_t a = tr_frag<T::kStride>(qtile + tr_base, ks, db * 64);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb[ks], dk[db], 0, 0, 0);
      }
    }
  }
  store_rows<D>(dKg + head, key, N, dk, scale, g);
  store_rows<D>(dVg + head, key, N, dv, 1.f, g);
}

// ---------------------------------------------------------------------------
// 3. dQ: one workgroup per kBwdQ queries of one head
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(const __bf16* __restrict__ Qg, const __bf16* __restrict__ Kg, const __bf16* __restrict__ Vg,
                   const __bf16* __restrict__ dOg, const float* __restrict__ Lg, const float* __restrict__ Dg,
                   __bf16* __restrict__ dQg, int N, int q_tiles, float scale) {
  using T = BwdTile<D>;
  // per buffer s: [K tile][V tile]
  __shared__ __attribute__((aligned(1024))) char smem[T::kDqLds];
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  char LDS_AS* lds = (char LDS_AS*)smem;
  auto kbuf = [&](int s) { return lds + s * 2 * T::kKTBytes; };
  auto vbuf = [&](int s) { return lds + s * 2 * T::kKTBytes + T::kKTBytes; };

  // work item: query tile qt of head bh, head-major over XCD-local logical
  // indices (a head's K and V tiles are re-read by all its query tiles, from
  // one L2); within a head the longest causal items (last query tiles) first
  const int lw = xcd_local_index(blockIdx.x, gridDim.x);
  const int bh = lw / q_tiles;
  const int r = lw - bh * q_tiles;
  const int qt = CAUSAL ? q_tiles - 1 - r : r;
  const size_t head = (size_t)bh * N * D;
  const unsigned head_bytes = (unsigned)N * D * 2;
  const int qw0 = qt * kBwdQ + wave * 32;  // first query of this wavefront
  const int qrow = qw0 + l32;              // this lane's query (column of every accumulator)

  // Q and dO rows of the lane's query as B operands; L (base 2) and D
  bf16x8_t qf[D / 16], dof[D / 16];
  float L2 = 0.f, Dq = 0.f;
  {
    const bf16x8_t* qp = reinterpret_cast<const bf16x8_t*>(Qg + head + (size_t)qrow * D) + g;
    const bf16x8_t* op = reinterpret_cast<const bf16x8_t*>(dOg + head + (size_t)qrow * D) + g;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      qf[ds] = qrow < N ? qp[2 * ds] : bf16x8_t{};
      dof[ds] = qrow < N ? op[2 * ds] : bf16x8_t{};
    }
    if (qrow < N) {
      L2 = Lg[(size_t)bh * N + qrow] * kLog2e;
      Dq = Dg[(size_t)bh * N + qrow];
    }
  }
  f32x16_t dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = f32x16_t{};

  // KV tiles: causal items stop at the last tile with a key <= their last query
  int n_kt = (N + kBwdKT - 1) / kBwdKT;
  if (CAUSAL) {
    const int last = min(N - 1, qt * kBwdQ + kBwdQ - 1);
    n_kt = min(n_kt, last / kBwdKT + 1);
  }
  const u32x4_t k_rsrc = make_rsrc(Kg + head, head_bytes);
  const u32x4_t v_rsrc = make_rsrc(Vg + head, head_bytes);
  auto issue = [&](int j, int s) {
    const unsigned soff = (unsigned)j * kBwdKT * T::kRowBytes;
    dma_rows(k_rsrc, soff, kbuf(s), T::kKTBytes, wave, lane, [](int o) { return padded_source<D>(o, true); });
    dma_rows(v_rsrc, soff, vbuf(s), T::kKTBytes, wave, lane, [](int o) { return padded_source<D>(o, true); });
  };

  const float c = scale * kLog2e;
  const int row_base = vrow_perm(l32) * T::kStride + g * 16;
  const int tr_base = tr_lane_base<T::kStride>(lane);
  constexpr int kKB = kBwdKT / 32;  // 32-key blocks per tile

  issue(0, 0);
  for (int j = 0; j < n_kt; ++j) {
    const int s = j & 1;
    wait_vmem();
    wg_barrier();
    if (j + 1 < n_kt) issue(j + 1, s ^ 1);
    const char LDS_AS* kb = kbuf(s);
    const char LDS_AS* vb = vbuf(s);
    const int k0 = j * kBwdKT;
    // every (query, key) pair of this wavefront's tile is valid: no per-element masks
    const bool full = k0 + kBwdKT <= N && qw0 + 32 <= N && (!CAUSAL || k0 + kBwdKT - 1 <= qw0);

    // S^T = K Q^T and dP^T = V dO^T (key rows, the lane's query in the column)
    f32x16_t sc[kKB], dp[kKB];
#pragma unroll
    for (int cb = 0; cb < kKB; ++cb) sc[cb] = dp[cb] = f32x16_t{};
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
#pragma unroll
      for (int cb = 0; cb < kKB; ++cb) {
        const bf16x8_t a = *(const bf16x8_t LDS_AS*)(kb + row_base + cb * 32 * T::kStride + ds * 32);
        sc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ds], sc[cb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
#pragma unroll
      for (int cb = 0; cb < kKB; ++cb) {
        const bf16x8_t a = *(const bf16x8_t LDS_AS*)(vb + row_base + cb * 32 * T::kStride + ds * 32);
        dp[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dof[ds], dp[cb], 0, 0, 0);
      }
    }
    // dS^T = P^T (dP^T - D), P^T = exp(S^T - L); keys past N and (causal)
    // keys after the query get 0.  Element i of block cb is key
    // k0 + 32 cb + 8 (i >> 2) + 4 g + (i & 3).
    bf16x8_t dsb[kBwdKT / 16];
    float dsf[kKB][16];
    if (full) {
#pragma unroll
      for (int cb = 0; cb < kKB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          dsf[cb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[cb][i], c, -L2)) * (dp[cb][i] - Dq);
    } else {
#pragma unroll
      for (int cb = 0; cb < kKB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kr = k0 + 32 * cb + 8 * (i >> 2) + 4 * g + (i & 3);
          const bool ok = kr < N && qrow < N && (!CAUSAL || kr <= qrow);
          const float p = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(sc[cb][i], c, -L2)) : 0.f;
          dsf[cb][i] = p * (dp[cb][i] - Dq);
        }
    }
#pragma unroll
    for (int cb = 0; cb < kKB; ++cb)
#pragma unroll
      for (int h = 0; h < 2; ++h) dsb[2 * cb + h] = to_bf16x8(&dsf[cb][8 * h]);
    // dQ^T += K^T dS^T (keys are the contraction index)
#pragma unroll
    for (int ks = 0; ks < kBwdKT / 16; ++ks) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8_t a = tr_frag<T::kStride>(kb + tr_base, ks, db * 64);
        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb[ks], dq[db], 0, 0, 0);
      }
    }
  }
  store_rows<D>(dQg + head, qrow, N, dq, scale, g);
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.H * a.N;
  constexpr int kRowsPerDotBlock = 4 * (64 / (D / 8));
  hipLaunchKernelGGL((bwd_dot_kernel<D>), dim3((unsigned)((rows + kRowsPerDotBlock - 1) / kRowsPerDotBlock)),
                     dim3(256), 0, stream, static_cast<const __bf16*>(a.O), static_cast<const __bf16*>(a.dO), a.L,
                     a.Dws, a.L2ws, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int bh = a.B * a.H;
  const int kv_tiles = (a.N + kBwdKV - 1) / kBwdKV;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)(bh * kv_tiles)), dim3(kThreads), 0, stream,
                     static_cast<const __bf16*>(a.Q), static_cast<const __bf16*>(a.K),
                     static_cast<const __bf16*>(a.V), static_cast<const __bf16*>(a.dO), a.L2ws, a.Dws,
                     static_cast<__bf16*>(a.dK), static_cast<__bf16*>(a.dV), a.N, kv_tiles, a.scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int q_tiles = (a.N + kBwdQ - 1) / kBwdQ;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)(bh * q_tiles)), dim3(kThreads), 0, stream,
                     static_cast<const __bf16*>(a.Q), static_cast<const __bf16*>(a.K),
                     static_cast<const __bf16*>(a.V), static_cast<const __bf16*>(a.dO), a.L, a.Dws,
                     static_cast<__bf16*>(a.dQ), a.N, q_tiles, a.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, int d, hipStream_t stream) {
  if (d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace fa
