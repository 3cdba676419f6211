// FlashAttention forward for bf16 Q/K/V on gfx950 (MI355X), head dimension
// 64 (d = 128 runs fa_fwd_bf16_asm.hip, 64 rows per wavefront).
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
//  * 8 wavefronts per workgroup, 32 query rows each (split-Q across
//    wavefronts, the work split of the FlashAttention-2 section of the blog):
//    the wavefronts share each K/V tile through LDS and never exchange
//    partial outputs.  One workgroup per compute unit, two wavefronts per
//    SIMD (wavefronts w and w+4 share a SIMD).
//  * Q is read once, straight from HBM into registers, already in the
//    operand layout of the score product; LDS holds only K and V tiles
//    (double-buffered, kFwdBC keys each).  At the end of a query tile the
//    output rows pass through the then idle K/V area, so that they leave as
//    whole rows (16 lanes per 256-byte row) rather than as 32 row pieces per
//    store instruction.
//  * Scores are formed transposed, S^T = K_j Q_i^T, on
//    v_mfma_f32_32x32x16_bf16.  In the 32x32 accumulator layout a lane holds
//    one query column and 16 key rows per 32-key block, so the softmax
//    reductions along keys are in-lane (v_max3_f32 chains and fp32 adds)
//    plus one v_permlane32_swap (lanes l and l^32 hold the two key halves of
//    the same query).
//  * The probabilities W leave the score accumulator already in the
//    B-operand layout of the second product U^T += V_j^T W^T, so W never
//    goes through LDS.  The matching A operand (8 keys of one head dimension
//    per lane) is assembled by two transposing LDS reads (ds_read_b64_tr_b16).
//  * K and V go from HBM to LDS with direct buffer->LDS loads (no staging
//    registers; rows past N read as zeros).  LDS rows are padded by 16 bytes,
//    and V rows are stored in a permuted order, so that every LDS read of the
//    loop (16-byte K fragments, transposing V reads) is free of bank
//    conflicts and addressed by one per-lane base register plus a
//    compile-time offset.
//  * Ping-pong schedule: each KV tile takes two slots per wavefront, a
//    softmax slot (VALU only) and a matrix slot (MFMA only: the W V product
//    of this tile, then the scores of the next).  The two wavefronts of a
//    SIMD run one slot apart, so the matrix core works on one wavefront's
//    products while the other computes its exponentials; a workgroup barrier
//    after every second slot (the one that also guards the K/V buffers)
//    keeps them in step.
//  * U^T lives in the accumulator layout with the query on the lane, so a
//    rescale by alpha is one multiply per register.  Rescaling is
//    conditional ("Infra: Flash Attention", section "Invariant of
//    conditional rescaling"): the base r of a row moves only when the tile
//    maximum exceeds it by more than 8 in the base-2 exponent, so W <= 2^8;
//    l, U and the new tile always share the same base and the final U / l is
//    unchanged.  Exponentials run in base 2 with scale*log2(e) folded into
//    one FMA per score.
//  * Workgroup ids are remapped so that all query tiles of one head run on
//    the same XCD (dispatch is round-robin over the 8 XCDs), letting the
//    head's K/V re-reads hit that XCD's L2; causal launches take the longest
//    query tiles of each head first.

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

using namespace dev;

constexpr float kRescaleLog2 = 8.f;  // conditional-rescale threshold (base-2 exponent)
constexpr int kThreads = kFwdWaves * 64;
constexpr int kKB = kFwdBC / 32;  // 32-key blocks per KV tile (score accumulators)
constexpr int kKS = kFwdBC / 16;  // 16-key MFMA steps per KV tile

// Tuning knob (compile-time).
#ifndef FA_FWD_PINGPONG
#define FA_FWD_PINGPONG 1  // 0: every wavefront in group 0 (lockstep slots)
#endif

// Issue order of the matrix slot's kR LDS reads (the transposing V reads,
// then the K-fragment reads) among its kM MFMAs: kUp = kR/4 reads first,
// then after MFMA i enough reads that kUp + (i+1)(kR - kUp)/kSpan have been
// issued, so the last read goes out after MFMA kSpan-1, kSpan = 5 kM / 8
// (12 and 20 of 48 reads and 32 MFMAs at d = 128; measured flat from 10 to
// 14 and from 16 to 22).  Left to itself the compiler issues the K reads of
// the next scores only after the last W.V product and then keeps two in
// flight, so the scores wait on LDS latency.
template <int I, int kM, int kR>
__device__ __forceinline__ void pin_matrix_steps() {
  constexpr int kUp = kR / 4, kSpan = 5 * kM / 8;
  if constexpr (I < kM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    constexpr int before = I < kSpan ? kUp + I * (kR - kUp) / kSpan : kR;
    constexpr int after = I + 1 < kSpan ? kUp + (I + 1) * (kR - kUp) / kSpan : kR;
    if constexpr (after > before) __builtin_amdgcn_sched_group_barrier(0x100, after - before, 0);  // LDS reads
    pin_matrix_steps<I + 1, kM, kR>();
  }
}
template <int kM, int kR>
__device__ __forceinline__ void pin_matrix_slot() {
  __builtin_amdgcn_sched_group_barrier(0x100, kR / 4, 0);
  pin_matrix_steps<0, kM, kR>();
}

template <int D>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kStride = kRowBytes + 16;           // padded LDS row
  static constexpr int kChunks = D / 8;                    // 16-byte chunks per row
  static constexpr int kBytes = kFwdBC * kStride;          // one K or V tile in LDS
  static constexpr int kLoads = kBytes / 1024;             // 1 KiB buffer->LDS loads per tile
  static constexpr int kLdsBytes = 4 * kBytes;             // K x2, V x2
  static constexpr int kLoadsPerWave = (kLoads + kFwdWaves - 1) / kFwdWaves;
  static_assert(kLoads * 1024 == kBytes, "padded tiles must be whole KiB");
  static_assert(kLdsBytes == fwd_lds_bytes(D), "LDS size must match the planner");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const __bf16* __restrict__ Qg, const __bf16* __restrict__ Kg,
                     const __bf16* __restrict__ Vg, __bf16* __restrict__ Og,
                     float* __restrict__ Lg, int N, int q_tiles, int units, float scale) {
  using T = Tile<D>;
  // [K buffer 0][K buffer 1][V buffer 0][V buffer 1], padded rows
  __shared__ __attribute__((aligned(1024))) char smem[T::kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;  // lane group: which 8-wide k slice a lane feeds

  char LDS_AS* lds = (char LDS_AS*)smem;
  auto kbuf = [&](int s) { return lds + s * T::kBytes; };
  auto vbuf = [&](int s) { return lds + (2 + s) * T::kBytes; };

  // ---- buffer -> LDS loads: per-lane offsets within a tile (the tile
  // offset is scalar)
  unsigned k_voff[T::kLoadsPerWave], v_voff[T::kLoadsPerWave];
#pragma unroll
  for (int p = 0; p < T::kLoadsPerWave; ++p) {
    const int o = (wave + p * kFwdWaves) * 1024 + lane * 16;
    k_voff[p] = padded_source<D>(o, false);
    v_voff[p] = padded_source<D>(o, true);
  }
  const unsigned head_bytes = (unsigned)N * D * 2;
  // one K or V tile through the head's resource, the tile offset in the SGPR
  // offset (range-checked on gfx950: rows past N read as zeros)
  auto dma_tile = [&](const u32x4_t rsrc, const unsigned* voff, int tile, char LDS_AS* dst) {
    const unsigned soff = (unsigned)tile * kFwdBC * T::kRowBytes;
#pragma unroll
    for (int p = 0; p < T::kLoadsPerWave; ++p) {
      const int blk = wave + p * kFwdWaves;
      if (p + 1 < T::kLoadsPerWave || blk < T::kLoads)
        load_lds16(rsrc, (void LDS_AS*)(dst + blk * 1024), voff[p], soff);
    }
  };

  // ---- per-lane LDS read bases (everything else is a compile-time offset)
  // K fragment (A operand of S^T = K Q^T): row l32, chunk 2*ds + g
  const int k_base = l32 * T::kStride + g * 16;
  // V^T fragment (A operand of U^T += V^T W^T) for head-dimension block db
  // and key step ks: two transposing reads of keys ks*16 + 8t + 4g + 0..3
  const int v_base = tr_lane_base<T::kStride>(lane);
  auto v_frag = [&](const char LDS_AS* vb, int db, int ks) { return tr_frag<T::kStride>(vb, ks, db * 64); };

  const float c = scale * kLog2e;
  const float theta = kRescaleLog2 / c;  // threshold in raw score units
  const int grp = FA_FWD_PINGPONG ? (wave >> 2) : 0;

  // ---- per-item state: Q fragments (B-operand layout of S^T = K Q^T: lane
  // (l32, g) holds Q[qrow][16 ds + 8 g + 0..7] for every d-step ds), the
  // online-softmax base m (raw score units, equal in lanes l and l^32), the
  // per-lane partial l over the lane's keys, and the U^T accumulators
  bf16x8_t qf[D / 16];
  float m_ref, l_run;
  f32x16_t u[D / 32];

  // KV tiles of query tile qt (causal tiles wholly in the future skipped)
  auto tiles_of = [&](int qt) {
    int n = (N + kFwdBC - 1) / kFwdBC;
    if (CAUSAL) {
      int last = qt * kFwdBR + kFwdBR - 1;
      if (last > N - 1) last = N - 1;
      n = min(n, last / kFwdBC + 1);
    }
    return n;
  };

  // ---- start of an item (query tile qt of head bh): Q into registers, and
  // K_0, V_0, K_1 into LDS.  Only issues loads; the item waits for them.
  auto start_q = [&](const int bh, const int qt) {
    const size_t head_off = (size_t)bh * N * D;
    const int qrow = qt * kFwdBR + wave * 32 + l32;
    // rows past N read as zeros; their outputs are never stored
    const bf16x8_t* qp = reinterpret_cast<const bf16x8_t*>(Qg + head_off + (size_t)qrow * D) + g;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) qf[ds] = bf16x8_t{};
    if (qrow < N) {
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) qf[ds] = qp[2 * ds];
    }
  };
  auto start_kv = [&](const int bh, const int qt) {
    const size_t head_off = (size_t)bh * N * D;
    const u32x4_t k_rsrc = make_rsrc(Kg + head_off, head_bytes);
    const u32x4_t v_rsrc = make_rsrc(Vg + head_off, head_bytes);
    dma_tile(k_rsrc, k_voff, 0, kbuf(0));
    dma_tile(v_rsrc, v_voff, 0, vbuf(0));
    if (tiles_of(qt) > 1) dma_tile(k_rsrc, k_voff, 1, kbuf(1));
  };

  // ---- one item: Algorithm 1 over its KV tiles, leaving (m, l, U).  Ends
  // with a workgroup barrier after which no wavefront reads this item's LDS.
  auto run_item = [&](const int bh, const int qt) {
  const size_t head_off = (size_t)bh * N * D;
  const int qw0 = qt * kFwdBR + wave * 32;  // first query row of this wavefront
  const int qrow = qw0 + l32;               // the query this lane's column belongs to
  const int n_tiles = tiles_of(qt);
  const u32x4_t k_rsrc = make_rsrc(Kg + head_off, head_bytes);
  const u32x4_t v_rsrc = make_rsrc(Vg + head_off, head_bytes);

  // S^T tile (kFwdBC keys x 32 queries) from the K tile at `kb`: block c of
  // 32 keys accumulates in s[cb]
  auto scores = [&](const char LDS_AS* kb, f32x16_t (&s)[kKB]) {
#pragma unroll
    for (int cb = 0; cb < kKB; ++cb) s[cb] = f32x16_t{};
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
#pragma unroll
      for (int cb = 0; cb < kKB; ++cb) {
        const bf16x8_t a = *(const bf16x8_t LDS_AS*)(kb + k_base + cb * 32 * T::kStride + ds * 32);
        s[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ds], s[cb], 0, 0, 0);
      }
    }
  };

  auto needs_mask = [&](int j) {
    const int kbase = j * kFwdBC;
    return (kbase + kFwdBC > N) || (CAUSAL && kbase + kFwdBC - 1 > qw0);
  };
  // keys past N, and keys after the query when causal, get -inf
  auto apply_mask = [&](int j, f32x16_t (&s)[kKB]) {
    const int kbase = j * kFwdBC;
    const int lim = CAUSAL ? min(N - 1, qrow) : N - 1;  // last valid key
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kr = kbase + 8 * (i >> 2) + 4 * g + (i & 3);
#pragma unroll
      for (int cb = 0; cb < kKB; ++cb)
        if (kr + 32 * cb > lim) s[cb][i] = -INFINITY;
    }
  };

  m_ref = -INFINITY;
  l_run = 0.f;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) u[db] = f32x16_t{};

  // ---- slot schedule.  The loop runs in slots; a workgroup barrier ends
  // every odd slot.  Each KV tile j takes two slots per wavefront: a softmax slot
  // (VALU only: W = exp2(c S_j - c m), l, rescale) and a matrix slot (MFMA
  // only: U^T += V_j^T W^T, then S_{j+1} = K_{j+1} Q^T).  Group 0 (waves
  // 0-3) runs tile j in slots 2j+1, 2j+2; group 1 (waves 4-7, the other
  // wavefront of each SIMD) one slot later, so in every slot one wavefront
  // per SIMD keeps the matrix core busy while the other runs the softmax.
  // Slot 0 forms S_0 everywhere; group 1 idles in slot 1.  Loads are issued
  // in even slots 2t (t >= 1): K_{t+1} and V_t, each into the buffer whose
  // last reader ran in slot 2t-1; they are waited for at the end of slot
  // 2t+1, before their first reader in slot 2t+2.  Those are the only
  // orderings the buffers need, so only odd slots end with a barrier (with
  // one after every slot, causal and non-causal prefill were 1-2 % slower).
  auto issue_slot = [&](int s) {
    if ((s & 1) == 0 && s >= 2) {
      const int t = s >> 1;
      if (t + 1 < n_tiles) dma_tile(k_rsrc, k_voff, t + 1, kbuf((t + 1) & 1));
      if (t < n_tiles) dma_tile(v_rsrc, v_voff, t, vbuf(t & 1));
    }
  };
  auto end_slot = [&](int s) {
    if (s & 1) {
      wait_vmem();
      wg_barrier();
    }
  };

  // ---- slot 0: the loads of start_q and start_kv have landed (and the
  // stores of the previous item's O are complete), S_0 everywhere
  wait_vmem();
  __syncthreads();
  f32x16_t s[kKB];  // scores of the current tile
  scores(kbuf(0), s);
  if (needs_mask(0)) apply_mask(0, s);
#pragma unroll
  for (int cb = 0; cb < kKB; ++cb) keep(s[cb]);
  end_slot(0);
  if (grp == 1) end_slot(1);  // group 1's idle slot

  for (int j = 0; j < n_tiles; ++j) {
    const int sa = 2 * j + 1 + grp;

    // -- softmax slot of tile j (VALU)
    issue_slot(sa);
    // row max: one chain per 32-key block, then across blocks and lane pairs
    float mxc[kKB];
#pragma unroll
    for (int cb = 0; cb < kKB; ++cb) {
      float m = fmaxf(s[cb][0], s[cb][1]);
#pragma unroll
      for (int i = 2; i < 16; i += 2) m = fmaxf(fmaxf(m, s[cb][i]), s[cb][i + 1]);
      mxc[cb] = m;
    }
    float mx = mxc[0];
#pragma unroll
    for (int cb = 1; cb < kKB; ++cb) mx = fmaxf(mx, mxc[cb]);
    mx = pair_max(mx);
    // move the base only if the tile max exceeds it by more than the
    // threshold (always on the first tile with a valid key)
    const float m_new = (mx > m_ref + theta) ? mx : m_ref;
    const float mc = (m_new == -INFINITY) ? 0.f : m_new * c;
    const bool moved = m_new > m_ref;
    const float alpha = moved ? __builtin_amdgcn_exp2f(m_ref * c - mc) : 1.f;
    m_ref = m_new;
    if (__any(moved)) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) u[db] *= alpha;
    }
    // W in bf16 for the product, fp32 partial sums for l (so l and L carry
    // no bf16 rounding): wb[2c + h] holds key step 2c + h
    bf16x8_t wb[2 * kKB];
    float rsp[2 * kKB];
#pragma unroll
    for (int cb = 0; cb < kKB; ++cb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float p[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) p[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[cb][8 * h + t], c, -mc));
        rsp[2 * cb + h] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        wb[2 * cb + h] = bf16x8_t{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                                 (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
      }
    }
#pragma unroll
    for (int w = 2 * kKB; w > 1; w >>= 1) {
#pragma unroll
      for (int i = 0; i < w / 2; ++i) rsp[i] += rsp[i + w / 2];
    }
    l_run = alpha * l_run + rsp[0];
    // keep the compiler from sinking the softmax into the matrix slot
#pragma unroll
    for (int k = 0; k < 2 * kKB; ++k) keep(wb[k]);
    keep(l_run);
    end_slot(sa);

    // -- matrix slot of tile j (MFMA): U^T += V_j^T W^T, then the scores of
    // tile j+1, as one straight-line block whose read/MFMA interleave is
    // pinned.  Both run unconditionally: a wavefront whose rows all precede
    // this tile's first key has W = 0 and adds exact zeros, and after the
    // last tile the scores of a stale K buffer are formed and never used.
    issue_slot(sa + 1);
    {
      const char LDS_AS* vb = vbuf(j & 1) + v_base;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
          const bf16x8_t a = v_frag(vb, db, ks);
          u[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, wb[ks], u[db], 0, 0, 0);
        }
      }
    }
    scores(kbuf((j + 1) & 1), s);
    pin_matrix_slot<2 * (D / 32) * kKS, 2 * (D / 32) * kKS + (D / 16) * kKB>();
    if (j + 1 < n_tiles && needs_mask(j + 1)) apply_mask(j + 1, s);
    // keep the products in this slot
#pragma unroll
    for (int cb = 0; cb < kKB; ++cb) keep(s[cb]);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) keep(u[db]);
    // every wavefront passes n_tiles barriers in the loop (odd slots 1, 3,
    // ..., 2 n_tiles - 1): group 1 has the extra idle slot 1, so it skips
    // the end of its final slot 2 n_tiles + 1
    if (!(grp == 1 && j == n_tiles - 1)) end_slot(sa + 1);
  }

  // every wavefront has finished reading this item's K/V tiles
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  wg_barrier();
  };

  // ---- end of an item: O = U / l, L = m * scale + ln l.  Called after
  // the item's last barrier, when no wavefront reads the K/V tiles any more:
  // O goes through the wavefront's own 32 padded rows of that area, in
  // which each lane writes its row's pieces; whole rows then leave with one
  // 16-byte store per lane, D/8 lanes per row.  (Stored straight from the
  // accumulator layout, every store instruction would touch 32 rows.)
  auto finish_item = [&](const int bh, const int qt) {
  const size_t head_off = (size_t)bh * N * D;
  const int qw0 = qt * kFwdBR + wave * 32;
  const int qrow = qw0 + l32;
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  char LDS_AS* const stage = lds + wave * 32 * T::kStride;
  // the lane index as an opaque copy, so that the lane-dependent addresses
  // below are formed here and not hoisted out of the item loop, where they
  // would hold registers across the tile loop
  int ln = lane;
  asm volatile("" : "+v"(ln));
  {
    // lane (l32, g) holds head dimensions db*32 + 8*i4 + 4*g + 0..3
    char LDS_AS* ob = stage + (ln & 31) * T::kStride + 8 * (ln >> 5);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        u32x2_t v;
        v[0] = pack_bf16x2(u[db][4 * i4 + 0] * inv, u[db][4 * i4 + 1] * inv);
        v[1] = pack_bf16x2(u[db][4 * i4 + 2] * inv, u[db][4 * i4 + 3] * inv);
        *(u32x2_t LDS_AS*)(ob + 64 * db + 16 * i4) = v;
      }
    }
  }
  // the rows are this wavefront's own, and LDS serves a wavefront in order
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  {
    constexpr int kRowsPer = 64 / T::kChunks;  // rows per store instruction
    const int rr = ln / T::kChunks, ch = ln % T::kChunks;
#pragma unroll
    for (int k = 0; k < 32 / kRowsPer; ++k) {
      const int r = k * kRowsPer + rr;
      const u32x4_t v = *(const u32x4_t LDS_AS*)(stage + r * T::kStride + ch * 16);
      if (qw0 + r < N) *reinterpret_cast<u32x4_t*>(Og + head_off + (size_t)(qw0 + r) * D + ch * 8) = v;
    }
  }
  if (Lg != nullptr && g == 0 && qrow < N) {
    Lg[(size_t)bh * N + qrow] = l_tot > 0.f ? m_ref * scale + __logf(l_tot) : -INFINITY;
  }
  // every wavefront has read its O rows back before K/V loads reuse the area
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  wg_barrier();
  };

  // ---- workgroup -> work units.  A unit is one query tile, or for causal
  // attention the pair of query tiles (p, q_tiles-1-p) of one head, so that
  // every causal unit has the same number of KV tiles.  Causal launches are
  // persistent: G workgroups (one per compute unit) take units logical(w),
  // logical(w) + G, ..., a static and balanced assignment that does not
  // depend on the order in which the hardware refills compute units.  Units
  // are numbered head-major and the logical index places consecutive units on
  // one XCD (dispatch is round-robin over the 8 XCDs), so the units running
  // at once on an XCD share heads and their K/V in L2.
  const int G = gridDim.x;
  const int wg = blockIdx.x;
  const int per = G >> 3, rem = G & 7;
  const int xcd = wg & 7, slot_id = wg >> 3;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + slot_id;
  if constexpr (CAUSAL) {
    // items in order: per unit the longer query tile, then the shorter one;
    // the next item's Q loads are issued before this item's O is stored, its
    // K/V loads after (O passes through the K/V area)
    const int pairs_per_head = (q_tiles + 1) >> 1;
    int unit = logical, second = 0;
    auto item_of = [&](int un, int sec, int& bh, int& qt) {
      bh = un / pairs_per_head;
      const int p = un - bh * pairs_per_head;
      qt = sec ? p : q_tiles - 1 - p;
    };
    int bh, qt;
    item_of(unit, second, bh, qt);
    start_q(bh, qt);
    start_kv(bh, qt);
    for (;;) {
      run_item(bh, qt);
      // advance: the shorter tile of this pair if it is distinct, else the
      // next unit
      const int p = unit - (unit / pairs_per_head) * pairs_per_head;
      if (second == 0 && p < q_tiles - 1 - p) {
        second = 1;
      } else {
        second = 0;
        unit += G;
      }
      const bool more = unit < units;
      int nbh = 0, nqt = 0;
      if (more) {
        item_of(unit, second, nbh, nqt);
        start_q(nbh, nqt);
      }
      finish_item(bh, qt);
      if (!more) break;
      start_kv(nbh, nqt);
      bh = nbh;
      qt = nqt;
    }
  } else {
    // one workgroup per query tile (the grid equals the unit count)
    const int bh = logical / q_tiles;
    const int qt = logical - bh * q_tiles;
    start_q(bh, qt);
    start_kv(bh, qt);
    run_item(bh, qt);
    finish_item(bh, qt);
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int q_tiles = (a.N + kFwdBR - 1) / kFwdBR;
  const int64_t units = fwd_units(a.B, a.H, a.N, a.causal);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)a.grid), dim3(kThreads), 0, stream,
                     static_cast<const __bf16*>(a.Q), static_cast<const __bf16*>(a.K),
                     static_cast<const __bf16*>(a.V), static_cast<__bf16*>(a.O), a.L, a.N, q_tiles,
                     (int)units, a.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, hipStream_t stream) {
  if (fwd_uses_asm(d, a.causal)) return launch_fwd_bf16_asm(a, stream);  // d = 128
  return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace fa
