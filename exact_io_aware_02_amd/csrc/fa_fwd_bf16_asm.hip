// FlashAttention forward for bf16 Q/K/V, d = 128, causal or not, on gfx950:
// 64 query rows per wavefront, one wavefront per SIMD, the tile loop in
// generated assembly.
//
// Same computation as fa_fwd_bf16.hip: Algorithm 1 of "Infra: Flash
// Attention" (section "Tiled computation and forward") in the
// FlashAttention-2 order of the "CMU 10-423 Lecture 18" notes (section 3.4),
// with conditional rescaling ("Invariant of conditional rescaling").  What
// differs is the split of the work on a compute unit:
//  * 4 wavefronts of 64 query rows (B_r = 256), one per SIMD.  Every K or V
//    fragment read from LDS feeds two 32-query MFMAs, so a KV tile costs half
//    the LDS reads per flop of the 32-rows-per-wavefront kernel.
//  * Inside a wavefront, tile step j overlaps U += V_{j-1}^T W_{j-1}^T and
//    S_{j+1} = K_{j+1} Q^T on the matrix core with the softmax of S_j on the
//    VALU (the FlashAttention-3 overlap of the blog's FA-3 section).  A
//    wavefront keeps issuing independent VALU work while its MFMAs run.
//  * The softmax of a tile forms no row max while the base holds: weights
//    relative to the current base are summed, and only a tile whose sum
//    exceeds 2^8 (so possibly a weight above the threshold) is redone with
//    its row max and a rescale of U and l.
//  * U^T (128 registers) and the Q fragments (64) live in AGPRs, two score
//    and two probability tiles in VGPRs.  The compiler cannot hold that many
//    values without spilling, so one query tile's loop is assembly generated
//    by gen_fwd_asm.py with one fixed register for every value.
//  * Causal: tiles wholly after a query tile are never visited; a
//    wavefront masks its diagonal tile, and skips the products of tiles
//    wholly after its 64 rows (inside the query tile's range), issuing only
//    its share of their loads and joining the barriers; a skipped tile's
//    softmax, where it still runs, gets zero weights through m c = +inf.
//  * Persistent workgroups, one per compute unit: during an item's last
//    product block the next item's Q fragments and first two K tiles load
//    into the registers and K buffers that block no longer reads, and the
//    output leaves through a staging area of its own, so consecutive items
//    do not wait for each other's loads or stores.

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_fwd_asm_d128.inc"

namespace fa {
namespace {

using namespace dev;

constexpr int D = 128;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBR = 64 * kWaves;
constexpr int kBC = 64;
constexpr int kStride = 2 * D + 16;
constexpr int kTile = kBC * kStride;
// [K buffer 0][K buffer 1][V buffer 0][V buffer 1][output staging: 64 rows
// per wavefront]; one workgroup fills a compute unit (160 KiB of LDS)
constexpr int kKV = 4 * kTile;
constexpr int kLds = kKV + kWaves * 64 * kStride;
static_assert(kBR == kFwdBR && kBC == kFwdBC, "tiles must match the planner");
static_assert(kKV == fwd_lds_bytes(D) && kLds == fwd_asm_lds_bytes(), "LDS size must match the planner");

// POLY: exponentials per 64 of a tile evaluated by a polynomial on the
// multiply-add units instead of v_exp_f32 (0, or one of the generator's
// shares)
template <bool CAUSAL, int POLY>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_bf16_asm_kernel(const __bf16* __restrict__ Qg, const __bf16* __restrict__ Kg,
                         const __bf16* __restrict__ Vg, __bf16* __restrict__ Og,
                         float* __restrict__ Lg, int N, int q_tiles, int units, float scale) {
  __shared__ __attribute__((aligned(1024))) char smem[kLds];
  char LDS_AS* lds = (char LDS_AS*)smem;
  const unsigned lds_base = (unsigned)(size_t)lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // per-lane buffer->LDS source offsets of this wavefront's 1 KiB blocks
  unsigned kvo[5], vvo[5];
#pragma unroll
  for (int p = 0; p < 5; ++p) {
    const int o = (wave + p * kWaves) * 1024 + lane * 16;
    kvo[p] = padded_source<D>(o, false);
    vvo[p] = padded_source<D>(o, true);
  }
  // LDS bases: K fragments, transposing V reads (V buffers start after the
  // two K buffers), this wavefront's 64 staging rows as written from the
  // accumulators (row l32 of a query block, 8 columns per lane group) and as
  // read for the stores (row lane / 16 + 4 k, 16 bytes at lane % 16)
  const unsigned kb = lds_base + l32 * kStride + g * 16;
  const unsigned vb = lds_base + 2 * kTile + tr_lane_base<kStride>(lane);
  const unsigned stage = lds_base + kKV + wave * 64 * kStride;
  const unsigned stg = stage + l32 * kStride + 8 * g;
  const unsigned srd = stage + (lane >> 4) * kStride + (lane & 15) * 16;
  const unsigned wbase = lds_base + wave * 1024;

  const float c = scale * kLog2e;
  const float theta = 8.f / c;  // conditional-rescale threshold, raw score units
  const unsigned head_bytes = (unsigned)N * D * 2;
  const int kv_tiles = (N + kBC - 1) / kBC;
  // causal diagonal tile: key c + 4 g against query l32
  const int dg = l32 - 4 * g;

  // persistent: G workgroups take units lw, lw + G, ... (lw: the workgroup's
  // logical index).  A unit is a query tile, or for causal attention the
  // pair of query tiles (p, q_tiles - 1 - p) of a head, the longer first, so
  // that every causal unit has the same number of KV tiles.  Dispatch is
  // round-robin over the 8 XCDs and lw places a contiguous run of workgroups
  // on one XCD, so the units running at once on an XCD belong to the same
  // heads and share K/V in that XCD's L2.
  const int G = gridDim.x;
  const int wg = blockIdx.x;
  const int per = G >> 3, rem = G & 7;
  const int xcd = wg & 7, slot_id = wg >> 3;
  const int lw = xcd * per + (xcd < rem ? xcd : rem) + slot_id;
  const int pairs = (q_tiles + 1) >> 1;
  auto item_of = [&](int unit, int second, int& bh, int& qt) {
    if (CAUSAL) {
      bh = unit / pairs;
      const int p = unit - bh * pairs;
      qt = second ? p : q_tiles - 1 - p;
    } else {
      bh = unit / q_tiles;
      qt = unit - bh * q_tiles;
    }
  };
  // the item after (unit, second) in this workgroup's sequence
  auto advance = [&](int& unit, int& second) {
    if (CAUSAL && second == 0) {
      const int p = unit - (unit / pairs) * pairs;
      if (p < q_tiles - 1 - p) {
        second = 1;
        return;
      }
    }
    second = 0;
    unit += G;
  };

  int unit = lw, second = 0;
  int pre = 0;
  while (unit < units) {
    int bh, qt;
    item_of(unit, second, bh, qt);
    int nunit = unit, nsecond = second;
    advance(nunit, nsecond);
    const bool more = nunit < units;
    int nbh = bh, nqt = qt;
    if (more) item_of(nunit, nsecond, nbh, nqt);

    const size_t head_off = (size_t)bh * N * D;
    const size_t nhead_off = (size_t)nbh * N * D;
    const int qw0 = __builtin_amdgcn_readfirstlane(qt * kBR + wave * 64);
    const int nqw0 = nqt * kBR + wave * 64;
    // KV tiles of the item (causal: those wholly after its last row skipped)
    const int n = CAUSAL ? min(kv_tiles, min(N - 1, qt * kBR + kBR - 1) / kBC + 1) : kv_tiles;
    // keys past the lane's last valid one (N - 1, or causal its query) are
    // masked: the loop compares key - 4 g against the limit - 4 g
    const int limg0 = (CAUSAL ? min(N - 1, qw0 + l32) : N - 1) - 4 * g;
    const int limg1 = (CAUSAL ? min(N - 1, qw0 + 32 + l32) : N - 1) - 4 * g;
    const u32x4_t q_rsrc = make_rsrc(Qg + head_off, head_bytes);
    const u32x4_t nq_rsrc = make_rsrc(Qg + nhead_off, more ? head_bytes : 0u);
    const u32x4_t o_rsrc = make_rsrc(Og + head_off, head_bytes);
    const u32x4_t l_rsrc = Lg != nullptr ? make_rsrc(Lg + (size_t)bh * N, (unsigned)N * 4) : make_rsrc(nullptr, 0u);
    // K and V head bases: the loop builds each tile's resource from them
    const unsigned long long ka = (unsigned long long)(Kg + head_off);
    const unsigned long long va = (unsigned long long)(Vg + head_off);
    const unsigned long long nka = (unsigned long long)(Kg + nhead_off);
    const unsigned klo = (unsigned)ka, khi = (unsigned)(ka >> 32) & 0xFFFFu;
    const unsigned vlo = (unsigned)va, vhi = (unsigned)(va >> 32) & 0xFFFFu;
    const unsigned nklo = (unsigned)nka, nkhi = (unsigned)(nka >> 32) & 0xFFFFu;
    const unsigned nhb = more ? head_bytes : 0u;
    const unsigned qvo = (unsigned)(qw0 + l32) * D * 2 + g * 16;
    const unsigned nqvo = (unsigned)(nqw0 + l32) * D * 2 + g * 16;
    const unsigned ovo = (unsigned)(qw0 + (lane >> 4)) * D * 2 + (lane & 15) * 16;
    const unsigned lvo = (unsigned)(qw0 + l32) * 4;
#define FA_ASM_OPERANDS                                                                                          \
  :                                                                                                              \
  : [kvo0] "v"(kvo[0]), [kvo1] "v"(kvo[1]), [kvo2] "v"(kvo[2]), [kvo3] "v"(kvo[3]), [kvo4] "v"(kvo[4]),           \
    [vvo0] "v"(vvo[0]), [vvo1] "v"(vvo[1]), [vvo2] "v"(vvo[2]), [vvo3] "v"(vvo[3]), [vvo4] "v"(vvo[4]),           \
    [qvo] "v"(qvo), [nqvo] "v"(nqvo), [kb] "v"(kb), [vb] "v"(vb), [stg] "v"(stg), [srd] "v"(srd), [ovo] "v"(ovo), \
    [lvo] "v"(lvo), [limg0] "v"(limg0), [limg1] "v"(limg1), [dg] "v"(dg), [c] "v"(c), [theta] "v"(theta),        \
    [qrsrc] "s"(q_rsrc), [nqrsrc] "s"(nq_rsrc), [orsrc] "s"(o_rsrc), [lrsrc] "s"(l_rsrc), [klo] "s"(klo),        \
    [khi] "s"(khi), [vlo] "s"(vlo), [vhi] "s"(vhi), [hb] "s"(head_bytes), [nklo] "s"(nklo), [nkhi] "s"(nkhi),    \
    [nhb] "s"(nhb), [n] "s"(n), [wave] "s"(wave), [wbase] "s"(wbase), [n_keys] "s"(N), [qw0] "s"(qw0),           \
    [pre] "s"(pre)
    if constexpr (POLY == 0) {
      if constexpr (CAUSAL)
        asm volatile(FA_ASM_ITEM_CAUSAL FA_ASM_OPERANDS : FA_ASM_CLOBBERS);
      else
        asm volatile(FA_ASM_ITEM FA_ASM_OPERANDS : FA_ASM_CLOBBERS);
    } else if constexpr (POLY == 4) {
      if constexpr (CAUSAL)
        asm volatile(FA_ASM_ITEM_CAUSAL_POLY4 FA_ASM_OPERANDS : FA_ASM_CLOBBERS_POLY);
      else
        asm volatile(FA_ASM_ITEM_POLY4 FA_ASM_OPERANDS : FA_ASM_CLOBBERS_POLY);
    } else if constexpr (POLY == 8) {
      if constexpr (CAUSAL)
        asm volatile(FA_ASM_ITEM_CAUSAL_POLY8 FA_ASM_OPERANDS : FA_ASM_CLOBBERS_POLY);
      else
        asm volatile(FA_ASM_ITEM_POLY8 FA_ASM_OPERANDS : FA_ASM_CLOBBERS_POLY);
    } else {
      static_assert(POLY == 16, "a share the generator builds");
      if constexpr (CAUSAL)
        asm volatile(FA_ASM_ITEM_CAUSAL_POLY16 FA_ASM_OPERANDS : FA_ASM_CLOBBERS_POLY);
      else
        asm volatile(FA_ASM_ITEM_POLY16 FA_ASM_OPERANDS : FA_ASM_CLOBBERS_POLY);
    }
#undef FA_ASM_OPERANDS
    pre = 1;
    unit = nunit;
    second = nsecond;
  }
  // the last item's stores (and its empty prefetch) complete before the
  // workgroup's LDS and registers are released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <bool CAUSAL, int POLY>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int q_tiles = (a.N + kBR - 1) / kBR;
  const int64_t units = fwd_units(a.B, a.H, a.N, a.causal);
  hipLaunchKernelGGL((fwd_bf16_asm_kernel<CAUSAL, POLY>), dim3((unsigned)a.grid), dim3(kThreads), 0, stream,
                     static_cast<const __bf16*>(a.Q), static_cast<const __bf16*>(a.K),
                     static_cast<const __bf16*>(a.V), static_cast<__bf16*>(a.O), a.L, a.N, q_tiles,
                     (int)units, a.scale);
  return hipGetLastError();
}

template <int POLY>
hipError_t launch_poly(const FwdArgs& a, hipStream_t stream) {
  return a.causal ? launch<true, POLY>(a, stream) : launch<false, POLY>(a, stream);
}

}  // namespace

hipError_t launch_fwd_bf16_asm(const FwdArgs& a, hipStream_t stream) {
  switch (a.exp2_poly) {
    case 4: return launch_poly<4>(a, stream);
    case 8: return launch_poly<8>(a, stream);
    case 16: return launch_poly<16>(a, stream);
    default: return launch_poly<0>(a, stream);
  }
}

}  // namespace fa
