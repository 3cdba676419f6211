// Flash-Decoding on gfx950: one query per (b, h) against a long KV cache.
//
// The airsota Flash-Decoding card (section 3, steps 1-3) splits the cached
// sequence into chunks, lets an independent workgroup compute each chunk's
// partial attention -- its output O^(k), maximum m^(k) and normaliser
// l^(k) -- and merges the partials with a log-sum-exp reduction kernel.
// "Infra: Flash Attention" ("Prefill and decode") notes that the merge of
// (m, l, u) states allows any order, so the chunks may be reduced as a tree.
//
// Split kernel, grid (num_splits, H, B), 4 wavefronts per workgroup:
//  * the cost is reading K and V from HBM (intensity about one FLOP per
//    byte), so there is no matrix-core work: each 16-byte load of a
//    wavefront covers 64 lanes x 16 B = 4 whole 256-byte key rows (d = 128),
//    i.e. 1 KiB of contiguous cache per instruction;
//  * a lane dots its 8 dims with the query's 8 dims (the query is pre-scaled
//    by scale*log2(e) so exponentials run in base 2), and the 16 lanes of a
//    row finish the dot with 4 DPP steps;
//  * each wavefront keeps the online state (m, l, u) of the keys it has read;
//    blocks of 16 keys per wavefront are read ahead of their use (two blocks
//    in flight).  Short blocks keep the kernel at 144 VGPRs, so a compute
//    unit could hold three wavefronts per SIMD; measured, they stream faster
//    than 32-key blocks at 288 registers (one wavefront per SIMD);
//  * at the end the four wavefronts' states are merged through LDS and the
//    partial (O^(k) = u / l, lse_k = m + ln l) is written: this pair carries
//    exactly the card's (O^(k), m^(k), l^(k)) since l^(k) e^{m^(k)} = e^{lse_k}.
//    An empty chunk writes (0, -inf).
// Combine kernel, grid (H, B): M = max_k lse_k, w_k = e^{lse_k - M},
// o = sum_k w_k O^(k) / sum_k w_k, lse = M + ln sum_k w_k.
//
// One launch (fa_decode_fused): the split kernel itself merges.  Each split
// workgroup publishes its partial and counts itself in a per-(b, h) counter;
// the workgroup that brings the count to S merges the S partials with the
// combine kernel's arithmetic (so the results are bit-identical) and resets
// the counter.  The merge order is free ("Prefill and decode"), so which
// workgroup is last does not matter.  Publishing to a workgroup that may run
// on another XCD takes an agent-scope release: one wavefront writes the
// partial and performs the release with the counting atomic (so the ordering
// is within one instruction stream); only the last workgroup acquires,
// before it reads.
//
// Paged caches ("CMU 10-423 Lecture 18" notes, section 7.3): the cache is a
// pool of blocks of 2^log2_bs tokens, [num_blocks, H, block_size, d], and a
// block table maps each sequence's logical block to a physical one.  The
// split kernel stages its chunk's physical block ids in LDS once; every row
// address is then pool + ((id * H + h) * block_size + key % block_size) * d.
// block_size >= 16 keeps the rows of one load instruction inside one block.
// Ids outside [0, num_blocks) are never dereferenced: their tokens are
// skipped as if masked.  Per-chunk partials and the combine are the same as
// for a contiguous cache, so identical keys give identical results.

#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kThreads = kDecWaves * 64;
constexpr int kUnroll = 4;  // 16-byte loads of K (and of V) per lane per block

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of LANES (8 or 16) lanes; every lane gets the sum.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror: lane i <- lane 7-i within 8
  if constexpr (LANES == 16) x += dpp<0x140>(x);  // row_mirror: i <- 15-i
  return x;
}

__device__ __forceinline__ void bf16x8_to_f32(const u32x4_t v, float* f) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f[2 * w] = __uint_as_float(v[w] << 16);
    f[2 * w + 1] = __uint_as_float(v[w] & 0xffff0000u);
  }
}

constexpr int kCombineThreads = 256;
constexpr int kMaxSplits = 4096;  // the host rejects larger split counts

// Block-wide max / sum over kCombineThreads threads (4 wavefronts).
template <bool MAX>
__device__ __forceinline__ float block_reduce(float x, float* red) {
  for (int off = 32; off > 0; off >>= 1) {
    const float y = __shfl_xor(x, off);
    x = MAX ? fmaxf(x, y) : x + y;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  x = red[0];
  for (int w = 1; w < kCombineThreads / 64; ++w) x = MAX ? fmaxf(x, red[w]) : x + red[w];
  return x;
}

// The merge of the S partials of (b, h) = bh by one workgroup of
// kCombineThreads threads: M = max_k lse_k, w_k = e^{lse_k - M},
// o = sum_k w_k O^(k) / sum_k w_k, lse = M + ln sum_k w_k.  w (kMaxSplits
// floats), red and osum are LDS.  The partials are read with plain loads
// (not through the read-only path): in one launch they were written by
// other workgroups of the same kernel.
template <int D>
__device__ __forceinline__ void combine_partials(const float* part_o, const float* part_lse, __bf16* og,
                                                 float* lse_out, size_t bh, int S, float* w, float* red,
                                                 float* osum) {
  const int t = threadIdx.x;
  const size_t base = bh * S;
  float M = -INFINITY;
  for (int k = t; k < S; k += kCombineThreads) M = fmaxf(M, part_lse[base + k]);
  M = block_reduce<true>(M, red);
  float sw = 0.f;
  for (int k = t; k < S; k += kCombineThreads) {
    const float lk = part_lse[base + k];
    const float wk = (M == -INFINITY || lk == -INFINITY) ? 0.f : __expf(lk - M);
    w[k] = wk;
    sw += wk;
  }
  sw = block_reduce<false>(sw, red);  // its barriers also publish w[]

  // column t % D, partials k = t / D, t / D + 256 / D, ...
  constexpr int kGroups = kCombineThreads / D;
  const int col = t % D;
  float o = 0.f;
  for (int k = t / D; k < S; k += kGroups) o = __builtin_fmaf(w[k], part_o[(base + k) * D + col], o);
  osum[t] = o;
  __syncthreads();
  if (t < D) {
    float acc = osum[t];
#pragma unroll
    for (int gi = 1; gi < kGroups; ++gi) acc += osum[t + gi * D];
    og[bh * D + t] = (__bf16)(sw > 0.f ? acc / sw : 0.f);
    if (lse_out != nullptr && t == 0) lse_out[bh] = (M == -INFINITY) ? -INFINITY : M + __logf(sw);
  }
}

// FUSED: publish the partial, count the split in counters[b * H + h], and
// merge if this workgroup completes the count (og, lse_out: the outputs).
template <int D, bool PAGED, bool FUSED = false>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const __bf16* __restrict__ qg, const __bf16* __restrict__ Kg, const __bf16* __restrict__ Vg,
    const int32_t* __restrict__ Lkv, float* part_o, float* part_lse,
    int H, int S, int capacity, float scale, const int32_t* __restrict__ table, int max_blocks,
    int log2_bs, int num_blocks, int* counters = nullptr, __bf16* og = nullptr, float* lse_out = nullptr) {
  static_assert(!FUSED || kThreads == kCombineThreads, "the merge runs on the split workgroup");
  constexpr int CPR = D / 8;        // lanes per key row (16-byte chunks per row)
  constexpr int KPI = 64 / CPR;     // key rows per wavefront load instruction
  constexpr int KPB = KPI * kUnroll;  // keys per wavefront block

  __shared__ long long red64[kThreads];
  __shared__ float wstate[kDecWaves][2];
  __shared__ __attribute__((aligned(16))) float wacc[kDecWaves][D];
  __shared__ int ids[PAGED ? kPagedIdsPerChunk : 1];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane % CPR;   // this lane's 8-dim slice
  const int kr = lane / CPR;  // this lane's row within a load instruction

  // sequence length and the start of (b, h) in the cache
  int len = Lkv[b];
  len = len < 0 ? 0 : len;
  size_t row0 = 0;
  if (PAGED) {
    const long long cap = (long long)max_blocks << log2_bs;
    len = len > cap ? (int)cap : len;
  } else if (capacity > 0) {
    len = len > capacity ? capacity : len;
    row0 = ((size_t)b * H + h) * (size_t)capacity;
  } else {
    // tokens of the sequences before b (packed layout)
    long long part = 0;
    for (int i = tid; i < b; i += kThreads) {
      int li = Lkv[i];
      part += li > 0 ? li : 0;
    }
    red64[tid] = part;
    __syncthreads();
    for (int s = kThreads / 2; s > 0; s >>= 1) {
      if (tid < s) red64[tid] += red64[tid + s];
      __syncthreads();
    }
    const long long prefix = red64[0];
    row0 = (size_t)prefix * H + (size_t)h * len;
  }

  const int chunk = decode_chunk_tokens(len, S);
  const int start = split * chunk;
  const int end = min(len, start + chunk);
  const size_t out = ((size_t)b * H + h) * S + split;
  if (!FUSED && start >= end) {
    for (int e = tid; e < D; e += kThreads) part_o[out * D + e] = 0.f;
    if (tid == 0) part_lse[out] = -INFINITY;
    return;
  }
  // (fused: an empty chunk reads nothing and publishes the partial (0, -inf)
  // like any other, so that it is counted)

  // query slice, pre-scaled into the base-2 domain
  float qv[8];
  {
    const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(qg + ((size_t)b * H + h) * D + c * 8);
    bf16x8_to_f32(raw, qv);
    const float cs = scale * kLog2e;
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] *= cs;
  }

  const __bf16* Kh = Kg + row0 * D;
  const __bf16* Vh = Vg + row0 * D;

  // paged: this chunk's physical block ids (the host bounds their count)
  const int e_first = start >> log2_bs;
  if (PAGED && start < end) {
    const int e_last = (end - 1) >> log2_bs;
    for (int e = e_first + tid; e <= e_last; e += kThreads) ids[e - e_first] = table[(size_t)b * max_blocks + e];
    __syncthreads();
  }

  float m = -INFINITY, l = 0.f;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;

  // blocks of KPB keys, dealt round-robin to the wavefronts; the next block
  // of this wavefront is loaded while the current one is consumed
  const int n_blocks = start < end ? (end - start + KPB - 1) / KPB : 0;

  // bit u of `valid` is cleared when load u's block id is out of range
  // (paged only); such keys score -inf
  auto load_block = [&](int blk, u32x4_t (&kk)[kUnroll], u32x4_t (&vv)[kUnroll], unsigned& valid) {
    const int kbase0 = start + blk * KPB;
    valid = (1u << kUnroll) - 1;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int key = kbase0 + u * KPI + kr;
      size_t row = (size_t)key;
      bool ok = true;
      if (PAGED) {
        // the KPI rows of load u lie in one block: key0 = kbase0 + u * KPI
        const int id = ids[((kbase0 + u * KPI) >> log2_bs) - e_first];
        ok = (unsigned)id < (unsigned)num_blocks;
        if (!ok) valid &= ~(1u << u);
        row = ((((size_t)(ok ? id : 0)) * H + h) << log2_bs) + (key & ((1 << log2_bs) - 1));
      }
      if (ok && key < end) {
        kk[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Kh + row * D + c * 8));
        vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Vh + row * D + c * 8));
      } else {
        kk[u] = u32x4_t{};
        vv[u] = u32x4_t{};
      }
    }
  };

  auto process_block = [&](int blk, const u32x4_t (&kk)[kUnroll], const u32x4_t (&vv)[kUnroll],
                           const unsigned valid) {
    const int kbase = start + blk * KPB + kr;
    float s[kUnroll];
    float mb = -INFINITY;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float kf[8];
      bf16x8_to_f32(kk[u], kf);
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) p = __builtin_fmaf(qv[e], kf[e], p);
      p = group_sum<CPR>(p);
      s[u] = (kbase + u * KPI < end && ((valid >> u) & 1u)) ? p : -INFINITY;
      mb = fmaxf(mb, s[u]);
    }
    // block maximum across the wavefront's rows
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1) mb = fmaxf(mb, __shfl_xor(mb, off));
    const float m_new = fmaxf(m, mb);  // -inf only while every key so far was skipped
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);  // 0 on the first block
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float p = __builtin_amdgcn_exp2f(s[u] - m_use);  // 0 for keys past the chunk
      ps += p;
      float vf[8];
      bf16x8_to_f32(vv[u], vf);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(p, vf[e], acc[e]);
    }
    l = alpha * l + ps;
    m = m_new;
  };

  u32x4_t ka[kUnroll], va[kUnroll], kn[kUnroll], vn[kUnroll];
  unsigned oka = 0, okn = 0;
  int blk = wave;
  if (blk < n_blocks) load_block(blk, ka, va, oka);
  for (; blk < n_blocks; blk += 2 * kDecWaves) {
    if (blk + kDecWaves < n_blocks) load_block(blk + kDecWaves, kn, vn, okn);
    process_block(blk, ka, va, oka);
    if (blk + kDecWaves >= n_blocks) break;
    if (blk + 2 * kDecWaves < n_blocks) load_block(blk + 2 * kDecWaves, ka, va, oka);
    process_block(blk + kDecWaves, kn, vn, okn);
  }

  // wavefront totals: sum over the row groups (lanes with the same slice c)
#pragma unroll
  for (int off = CPR; off < 64; off <<= 1) {
    l += __shfl_xor(l, off);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off);
  }
  if (lane < CPR) {
#pragma unroll
    for (int e = 0; e < 8; ++e) wacc[wave][c * 8 + e] = acc[e];
  }
  if (lane == 0) {
    wstate[wave][0] = m;
    wstate[wave][1] = l;
  }
  __syncthreads();

  // merge the wavefronts' states (base-2 domain) and write the partial
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, wstate[w][0]);
  float f[kDecWaves];
  float L2 = 0.f;
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) {
    const float mw = wstate[w][0];
    f[w] = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
    L2 += f[w] * wstate[w][1];
  }
  // a chunk whose keys were all skipped (paged, invalid ids) is empty
  const float inv = L2 > 0.f ? 1.f / L2 : 0.f;
  if constexpr (!FUSED) {
    for (int e = tid; e < D; e += kThreads) {
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) o += f[w] * wacc[w][e];
      part_o[out * D + e] = o * inv;
    }
    if (tid == 0) part_lse[out] = L2 > 0.f ? (M + __log2f(L2)) * kLn2 : -INFINITY;
  } else {
    __shared__ int last;
    __shared__ float cw[kMaxSplits];
    __shared__ float cred[kCombineThreads / 64];
    __shared__ float cosum[kCombineThreads];
    const size_t bh = (size_t)b * H + h;
    if (wave == 0) {
      // the same values as the two-launch path, written by this wavefront
      // alone, which then releases them with the count
      for (int e = lane; e < D; e += 64) {
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) o += f[w] * wacc[w][e];
        part_o[out * D + e] = o * inv;
      }
      if (lane == 0) {
        part_lse[out] = L2 > 0.f ? (M + __log2f(L2)) * kLn2 : -INFINITY;
        // release only: the workgroups that are not last need no acquire
        const int prev = __hip_atomic_fetch_add(&counters[bh], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        last = prev == S - 1;
        // the last one acquires here: its atomic read the value of the
        // release sequence of every other split's count
        if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      }
    }
    __syncthreads();
    if (!last) return;
    // every partial of (b, h) is published: acquire (in every thread, after
    // the barrier that orders them after thread 0's acquire), reset the
    // counter for the next call, merge
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (tid == 0) __hip_atomic_store(&counters[bh], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    combine_partials<D>(part_o, part_lse, og, lse_out, bh, S, cw, cred, cosum);
  }
}

template <int D>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, __bf16* __restrict__ og,
    float* __restrict__ lse_out, int H, int S) {
  __shared__ float w[kMaxSplits];
  __shared__ float red[kCombineThreads / 64];
  __shared__ float osum[kCombineThreads];
  const int h = blockIdx.x, b = blockIdx.y;
  combine_partials<D>(part_o, part_lse, og, lse_out, (size_t)b * H + h, S, w, red, osum);
}

template <int D>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
  if (a.counters != nullptr) {
    hipLaunchKernelGGL((decode_split_kernel<D, false, true>), dim3(a.S, a.H, a.B), dim3(kThreads), 0, stream,
                       static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.K),
                       static_cast<const __bf16*>(a.V), a.Lkv, a.part_o, a.part_lse, a.H, a.S, a.capacity,
                       a.scale, nullptr, 0, 0, 0, a.counters, static_cast<__bf16*>(a.o), a.lse_out);
    return hipGetLastError();
  }
  if (a.table != nullptr)
    hipLaunchKernelGGL((decode_split_kernel<D, true>), dim3(a.S, a.H, a.B), dim3(kThreads), 0, stream,
                       static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.K),
                       static_cast<const __bf16*>(a.V), a.Lkv, a.part_o, a.part_lse, a.H, a.S, 0,
                       a.scale, a.table, a.max_blocks, a.log2_bs, a.num_blocks);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, false>), dim3(a.S, a.H, a.B), dim3(kThreads), 0, stream,
                       static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.K),
                       static_cast<const __bf16*>(a.V), a.Lkv, a.part_o, a.part_lse, a.H, a.S,
                       a.capacity, a.scale, nullptr, 0, 0, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.H, a.B), dim3(kCombineThreads), 0, stream, a.part_o,
                     a.part_lse, static_cast<__bf16*>(a.o), a.lse_out, a.H, a.S);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int d, hipStream_t stream) {
  return d == 128 ? launch<128>(a, stream) : launch<64>(a, stream);
}

}  // namespace fa
