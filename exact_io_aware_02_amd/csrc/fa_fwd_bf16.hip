// FlashAttention forward for bf16 Q/K/V on gfx950 (MI355X).
//
// What it computes is Algorithm 1 of "Infra: Flash Attention" (section
// "Tiled computation and forward"), in the FlashAttention-2 order of the
// "CMU 10-423 Lecture 18" notes (section 3.4): a workgroup owns one query
// tile of kFwdBR rows and walks the KV tiles; the per-row state (m, l, U)
// stays on chip and O = U / l is formed once at the end, with
// L = m + log l ("Backward and recomputation").  Causal tiles wholly in the
// future are never visited and diagonal tiles are masked on chip
// ("Infra: Flash Attention", causal figure; lecture notes section 4.3).
//
// Mapping onto CDNA4:
//  * 4 wavefronts per workgroup, 32 query rows each (split-Q across
//    wavefronts, the work split of the FlashAttention-2 section of the blog):
//    the wavefronts share each K/V tile through LDS and never exchange
//    partial outputs.
//  * Scores are formed transposed, S^T = K_j Q_i^T, with
//    v_mfma_f32_32x32x16_bf16.  In the 32x32 accumulator layout a lane holds
//    one query column and 16 key rows, so the softmax reductions along keys
//    are 31 in-lane max/add operations plus one exchange between lanes l and
//    l^32 (which hold the two key halves of the same query).
//  * The probabilities W leave the score accumulator already in the
//    B-operand layout of the second product U^T += V_j^T W^T, so W never
//    goes through LDS.  V_j is staged in LDS transposed (d-major) with its
//    keys permuted to match the accumulator's register order, so each
//    A-operand fragment is one 16-byte LDS read.
//  * U^T lives in the accumulator layout with the query on the lane, so the
//    rescale by alpha is one multiply per register with a per-lane scalar;
//    it is skipped when no row of the wavefront raised its maximum (alpha is
//    then exactly 1).
//  * Exponentials run in base 2: scale*log2(e) is folded into one FMA per
//    score before v_exp_f32.
//  * K/V tiles are double-buffered in LDS: the next tile's global loads are
//    in flight while the current tile is computed.  16-byte LDS chunks are
//    XOR-swizzled so the 16-byte reads and writes are bank-conflict free.
//  * Workgroup ids are remapped so that all query tiles of one head run on
//    the same XCD (dispatch is round-robin over the 8 XCDs), letting the
//    head's K/V re-reads hit that XCD's L2; causal launches take the longest
//    query tiles of each head first.

#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = kFwdWaves * 64;

template <int D>
struct Tile {
  static constexpr int kChunks = D / 8;                    // 16-byte chunks per K row
  static constexpr int kKBytes = kFwdBC * D * 2;           // K tile [BC][D]
  static constexpr int kVtRowBytes = kFwdBC * 2;           // Vt row: BC keys
  static constexpr int kVBytes = D * kVtRowBytes;          // Vt tile [D][BC]
  static constexpr int kBufBytes = kKBytes + kVBytes;
  static constexpr int kKLoads = kFwdBC * kChunks / kThreads;  // 16B loads per thread
  static constexpr int kKeysPerThreadV = kKLoads;              // V: keys per thread
  static_assert(kKLoads * kThreads == kFwdBC * kChunks, "tile/thread mismatch");
};

// Byte offset of 16-byte chunk `c` of K row `r` (XOR swizzle on r mod 8).
template <int D>
__device__ __forceinline__ int k_off(int r, int c) {
  return r * (D * 2) + ((c ^ (r & 7)) << 4);
}

// Byte offset of 16-byte chunk `c` of Vt row `dr`.  The swizzle mixes bits of
// dr and dr/8 so that both the reads (32 consecutive rows, same chunk) and
// the transposing writes (rows 8 apart, same chunk) spread over banks.
__device__ __forceinline__ int vt_off(int dr, int c) {
  return dr * (kFwdBC * 2) + ((c ^ ((dr ^ (dr >> 3)) & 7)) << 4);
}

// Position of key `k` inside a Vt row.  Within every group of 16 keys the
// second and third runs of 4 are swapped, which makes the 8 keys that one
// lane group feeds to one W^T V^T k-step contiguous.
__device__ __forceinline__ int vt_pos(int k) {
  int q4 = (k >> 2) & 3;
  int q4p = ((q4 & 1) << 1) | (q4 >> 1);
  return (k & ~15) | (q4p << 2) | (k & 3);
}

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, v);
}

// Value held by lane l^32 (the other key half of the same query).
__device__ __forceinline__ float swap32(float x) { return __shfl_xor(x, 32); }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const __bf16* __restrict__ Qg, const __bf16* __restrict__ Kg,
                     const __bf16* __restrict__ Vg, __bf16* __restrict__ Og,
                     float* __restrict__ Lg, int N, int q_tiles, float scale) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * T::kBufBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;  // lane group: which 8-wide k slice a lane feeds

  // ---- workgroup -> (head, query tile): XCD-aware, longest first if causal
  const int nb = gridDim.x;
  const int wg = blockIdx.x;
  const int per = nb >> 3, rem = nb & 7;
  const int xcd = wg & 7, slot = wg >> 3;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + slot;
  const int bh = logical / q_tiles;
  const int qi = logical - bh * q_tiles;
  const int qt = CAUSAL ? (q_tiles - 1 - qi) : qi;

  const size_t head_off = (size_t)bh * N * D;
  const __bf16* Qh = Qg + head_off;
  const __bf16* Kh = Kg + head_off;
  const __bf16* Vh = Vg + head_off;

  const int q0 = qt * kFwdBR;
  const int qw0 = q0 + wave * 32;  // first query row of this wavefront
  const int qrow = qw0 + l32;      // the query this lane's column belongs to

  int n_tiles = (N + kFwdBC - 1) / kFwdBC;
  if (CAUSAL) {
    int last = q0 + kFwdBR - 1;
    if (last > N - 1) last = N - 1;
    n_tiles = min(n_tiles, last / kFwdBC + 1);
  }

  // ---- Q fragments (B operand of S^T = K Q^T), kept in registers
  bf16x8_t qf[D / 16];
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds) {
    if (qrow < N) {
      qf[ds] = *reinterpret_cast<const bf16x8_t*>(Qh + (size_t)qrow * D + ds * 16 + g * 8);
    } else {
      qf[ds] = bf16x8_t{};
    }
  }

  // ---- staging registers for the next K/V tile
  u32x4_t kreg[T::kKLoads];
  u32x4_t vreg[T::kKeysPerThreadV];
  const int kc = tid % T::kChunks;  // chunk column this thread loads
  const int krow0 = tid / T::kChunks;
  constexpr int kRowsPerPass = kThreads / T::kChunks;
  const int vkey0 = (tid / T::kChunks) * T::kKeysPerThreadV;  // first of this thread's V keys

  auto load_tile = [&](int j) {
    const int kbase = j * kFwdBC;
#pragma unroll
    for (int p = 0; p < T::kKLoads; ++p) {
      int r = kbase + krow0 + p * kRowsPerPass;
      kreg[p] = (r < N) ? *reinterpret_cast<const u32x4_t*>(Kh + (size_t)r * D + kc * 8) : u32x4_t{};
    }
#pragma unroll
    for (int p = 0; p < T::kKeysPerThreadV; ++p) {
      int r = kbase + vkey0 + p;
      vreg[p] = (r < N) ? *reinterpret_cast<const u32x4_t*>(Vh + (size_t)r * D + kc * 8) : u32x4_t{};
    }
  };

  auto store_tile = [&](int buf) {
    char* kb = smem + buf * T::kBufBytes;
    char* vb = kb + T::kKBytes;
#pragma unroll
    for (int p = 0; p < T::kKLoads; ++p) {
      int r = krow0 + p * kRowsPerPass;
      *reinterpret_cast<u32x4_t*>(kb + k_off<D>(r, kc)) = kreg[p];
    }
    // transpose: thread holds keys vkey0.. (kKeysPerThreadV of them) x 8 dims
    const int pos = vt_pos(vkey0);
    const int cpos = pos >> 3;              // 16B chunk within the Vt row
    const int bpos = (pos & 7) * 2;         // byte within the chunk
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int dr = kc * 8 + e;
      char* dst = vb + vt_off(dr, cpos) + bpos;
      const int w = e >> 1;
      if constexpr (T::kKeysPerThreadV == 4) {
        unsigned a0 = vreg[0][w], a1 = vreg[1][w], a2 = vreg[2][w], a3 = vreg[3][w];
        u32x2_t out;
        if (e & 1) {
          out[0] = (a0 >> 16) | (a1 & 0xffff0000u);
          out[1] = (a2 >> 16) | (a3 & 0xffff0000u);
        } else {
          out[0] = (a0 & 0xffffu) | (a1 << 16);
          out[1] = (a2 & 0xffffu) | (a3 << 16);
        }
        *reinterpret_cast<u32x2_t*>(dst) = out;
      } else {
        unsigned a0 = vreg[0][w], a1 = vreg[1][w];
        unsigned out = (e & 1) ? ((a0 >> 16) | (a1 & 0xffff0000u)) : ((a0 & 0xffffu) | (a1 << 16));
        *reinterpret_cast<unsigned*>(dst) = out;
      }
    }
  };

  // ---- online-softmax state: m (raw score units, same in lanes l, l^32),
  // per-lane partial l over the lane's own keys, and U^T accumulators.
  const float c = scale * kLog2e;
  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16_t u[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) u[db] = f32x16_t{};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_tiles) load_tile(j + 1);

    const int kbase = j * kFwdBC;
    // a wavefront whose every row lies before this tile's first key has
    // nothing to add (all its rows are fully masked here): skip the update
    const bool wave_live = !CAUSAL || (kbase <= qw0 + 31);
    if (wave_live) {
      const char* kb = smem + buf * T::kBufBytes;
      const char* vb = kb + T::kKBytes;

      // S^T (keys x queries) for the two 32-key halves of the tile
      f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{};
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
        bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(kb + k_off<D>(l32, 2 * ds + g));
        bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(kb + k_off<D>(32 + l32, 2 * ds + g));
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ds], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ds], s1, 0, 0, 0);
      }

      // mask: keys past N, and keys after the query when causal
      const bool need_mask = (kbase + kFwdBC > N) || (CAUSAL && kbase + kFwdBC - 1 > qw0);
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kr = 8 * (i >> 2) + 4 * g + (i & 3);
          const int k0 = kbase + kr, k1 = kbase + 32 + kr;
          if (k0 >= N || (CAUSAL && k0 > qrow)) s0[i] = -INFINITY;
          if (k1 >= N || (CAUSAL && k1 > qrow)) s1[i] = -INFINITY;
        }
      }

      // row max over the tile's keys: in-lane, then across the lane pair
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
      mx = fmaxf(mx, swap32(mx));
      const float m_new = fmaxf(m_run, mx);
      // a row with no valid key so far keeps m = -inf: use base 0 so no
      // -inf - (-inf) is formed; its weights are exp2(-inf) = 0
      const float mc = (m_new == -INFINITY) ? 0.f : m_new * c;
      const bool raised = m_new > m_run;
      const float alpha = raised ? __builtin_amdgcn_exp2f(m_run * c - mc) : 1.f;

      // W = exp2(S*c - m'*c), row sums, and the bf16 B operands of W^T
      bf16x8_t wb[4];
      float rs = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float p[8], q[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          p[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[8 * h + t], c, -mc));
          q[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[8 * h + t], c, -mc));
          rs += p[t] + q[t];
        }
        wb[h] = bf16x8_t{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                         (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
        wb[2 + h] = bf16x8_t{(__bf16)q[0], (__bf16)q[1], (__bf16)q[2], (__bf16)q[3],
                             (__bf16)q[4], (__bf16)q[5], (__bf16)q[6], (__bf16)q[7]};
      }
      l_run = alpha * l_run + rs;

      // U = alpha U, skipped when no row of the wavefront raised its max
      if (__any(raised)) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) u[db] *= alpha;
      }

      // U^T += V^T W^T: k-steps of 16 keys, kstep = 2*kb + h
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int dr = db * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(vb + vt_off(dr, 2 * ks + g));
          u[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, wb[ks], u[db], 0, 0, 0);
        }
      }
      m_run = m_new;
    }

    if (j + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = U / l, L = m * scale + ln l
  const float l_tot = l_run + swap32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < N) {
    __bf16* orow = Og + head_off + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = db * 32 + 8 * i4 + 4 * g;
        u32x2_t v;
        v[0] = pack_bf16x2(u[db][4 * i4 + 0] * inv, u[db][4 * i4 + 1] * inv);
        v[1] = pack_bf16x2(u[db][4 * i4 + 2] * inv, u[db][4 * i4 + 3] * inv);
        *reinterpret_cast<u32x2_t*>(orow + d0) = v;
      }
    }
    if (Lg != nullptr && g == 0) {
      Lg[(size_t)bh * N + qrow] = l_tot > 0.f ? m_run * scale + __logf(l_tot) : -INFINITY;
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int q_tiles = (a.N + kFwdBR - 1) / kFwdBR;
  const int64_t nb = (int64_t)a.B * a.H * q_tiles;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)nb), dim3(kThreads), 0, stream,
                     static_cast<const __bf16*>(a.Q), static_cast<const __bf16*>(a.K),
                     static_cast<const __bf16*>(a.V), static_cast<__bf16*>(a.O), a.L, a.N, q_tiles,
                     a.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, hipStream_t stream) {
  if (d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace fa
