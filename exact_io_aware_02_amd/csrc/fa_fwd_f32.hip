// FlashAttention forward for fp32 Q/K/V on gfx950, every step in fp32.
//
// Algorithm 1 of "Infra: Flash Attention" (section "Tiled computation and
// forward") with B_r = B_c = 64: a workgroup owns 64 query rows and walks K_j
// and V_j tiles of 64 keys staged in LDS; every row keeps its (m, l, u)
// state in registers.  For each tile: S = Q K_j^T scale, a row whose keys
// are all masked in this tile skips the update ("Notation and boundary
// conditions"), otherwise m' = max(m, rowmax S), alpha = e^{(m - m') scale},
// W = e^{(S - m') scale}, l = alpha l + rowsum W, u = alpha u + W V_j.  At the
// end O = u / l and L = m scale + ln l.
//
// This path serves an fp32-input workload checked to 1e-5, so it stays on
// plain fp32 VALU FMAs (no reduced-precision matrix path).  Work split: four
// wavefronts of 16 rows, four lanes per row.  Lane quarter qq of a row forms
// the scores of keys 4 k + qq (so the four lanes read four consecutive,
// bank-disjoint K rows and the row groups of a wavefront share them by
// broadcast), the row max and sum are finished with two lane exchanges, the
// row's W goes through LDS, and the lane accumulates the output columns of
// 16-byte chunks 4 i + qq (again four bank-disjoint chunks per row).

#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kF32Threads = 256;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF32Threads) void fwd_f32_kernel(const float* __restrict__ Qg,
                                                               const float* __restrict__ Kg,
                                                               const float* __restrict__ Vg,
                                                               float* __restrict__ Og, float* __restrict__ Lg,
                                                               int N, int q_tiles, float scale) {
  static_assert(kF32BR == 64 && kF32BC == 64, "four wavefronts of 16 rows cover the tile");
  constexpr int kRow = D + 4;  // padded LDS row of K and V (floats): 4 banks apart
  constexpr int kPRow = kF32BC + 4;
  constexpr int kC = D / 16;   // 16-byte output chunks per lane
  __shared__ __attribute__((aligned(16))) float Ks[kF32BC * kRow];
  __shared__ __attribute__((aligned(16))) float Vs[kF32BC * kRow];
  __shared__ __attribute__((aligned(16))) float Ps[kF32BR * kPRow];

  const int tid = threadIdx.x;
  const int qq = tid & 3;          // quarter of the row
  const int rl = tid >> 2;         // row within the tile (0..63)
  const int bh = blockIdx.x / q_tiles;
  const int qt = blockIdx.x - bh * q_tiles;
  const size_t head_off = (size_t)bh * N * D;
  const int qrow = qt * kF32BR + rl;

  float q[D];
#pragma unroll
  for (int e = 0; e < D; e += 4) {
    const float4 v = qrow < N ? *reinterpret_cast<const float4*>(Qg + head_off + (size_t)qrow * D + e)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
    q[e] = v.x;
    q[e + 1] = v.y;
    q[e + 2] = v.z;
    q[e + 3] = v.w;
  }

  int n_tiles = (N + kF32BC - 1) / kF32BC;
  if (CAUSAL) {
    int last = qt * kF32BR + kF32BR - 1;
    if (last > N - 1) last = N - 1;
    n_tiles = min(n_tiles, last / kF32BC + 1);
  }

  float m = -INFINITY, l = 0.f;
  float u[kC][4];
#pragma unroll
  for (int c = 0; c < kC; ++c) u[c][0] = u[c][1] = u[c][2] = u[c][3] = 0.f;

  for (int j = 0; j < n_tiles; ++j) {
    const int kbase = j * kF32BC;
    __syncthreads();  // the previous tile's K, V and W are no longer read
    for (int idx = tid; idx < kF32BC * D / 4; idx += kF32Threads) {
      const int r = idx / (D / 4), c4 = (idx - r * (D / 4)) * 4;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (kbase + r < N) {
        kv = *reinterpret_cast<const float4*>(Kg + head_off + (size_t)(kbase + r) * D + c4);
        vv = *reinterpret_cast<const float4*>(Vg + head_off + (size_t)(kbase + r) * D + c4);
      }
      *reinterpret_cast<float4*>(&Ks[r * kRow + c4]) = kv;
      *reinterpret_cast<float4*>(&Vs[r * kRow + c4]) = vv;
    }
    __syncthreads();

    // scores of keys 4 k + qq
    float s[kF32BC / 4];
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kF32BC / 4; ++k) {
      const int kr = 4 * k + qq;
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < D; e += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(&Ks[kr * kRow + e]);
        acc = fmaf(q[e], kv.x, acc);
        acc = fmaf(q[e + 1], kv.y, acc);
        acc = fmaf(q[e + 2], kv.z, acc);
        acc = fmaf(q[e + 3], kv.w, acc);
      }
      const int key = kbase + kr;
      s[k] = key < N && (!CAUSAL || key <= qrow) ? acc : -INFINITY;
      mx = fmaxf(mx, s[k]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    // a row with every key of this tile masked skips the update: W = 0,
    // alpha = 1 (the same in its four lanes)
    const bool any = mx != -INFINITY;
    const float m_new = any ? fmaxf(m, mx) : m;
    const float alpha = !any ? 1.f : (m == -INFINITY ? 0.f : expf((m - m_new) * scale));
    float rs = 0.f;
#pragma unroll
    for (int k = 0; k < kF32BC / 4; ++k) {
      const float p = any ? expf((s[k] - m_new) * scale) : 0.f;  // exp(-inf) = 0 for masked keys
      rs += p;
      Ps[rl * kPRow + 4 * k + qq] = p;
    }
    rs += __shfl_xor(rs, 1);
    rs += __shfl_xor(rs, 2);
    l = alpha * l + rs;
    m = m_new;
    __syncthreads();  // the row's W is in LDS

    // u = alpha u + W V_j over the lane's 16-byte chunks 4 i + qq
#pragma unroll
    for (int c = 0; c < kC; ++c) u[c][0] *= alpha, u[c][1] *= alpha, u[c][2] *= alpha, u[c][3] *= alpha;
#pragma unroll 4
    for (int k = 0; k < kF32BC; k += 4) {
      const float4 p4 = *reinterpret_cast<const float4*>(&Ps[rl * kPRow + k]);
      const float pk[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int c = 0; c < kC; ++c) {
          const float4 vv = *reinterpret_cast<const float4*>(&Vs[(k + t) * kRow + 4 * (4 * c + qq)]);
          u[c][0] = fmaf(pk[t], vv.x, u[c][0]);
          u[c][1] = fmaf(pk[t], vv.y, u[c][1]);
          u[c][2] = fmaf(pk[t], vv.z, u[c][2]);
          u[c][3] = fmaf(pk[t], vv.w, u[c][3]);
        }
      }
    }
  }

  if (qrow < N) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int c = 0; c < kC; ++c)
      *reinterpret_cast<float4*>(Og + head_off + (size_t)qrow * D + 4 * (4 * c + qq)) =
          make_float4(u[c][0] * inv, u[c][1] * inv, u[c][2] * inv, u[c][3] * inv);
    if (Lg != nullptr && qq == 0) Lg[(size_t)bh * N + qrow] = l > 0.f ? m * scale + logf(l) : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int q_tiles = (a.N + kF32BR - 1) / kF32BR;
  const int64_t nb = (int64_t)a.B * a.H * q_tiles;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)nb), dim3(kF32Threads), 0, stream,
                     static_cast<const float*>(a.Q), static_cast<const float*>(a.K),
                     static_cast<const float*>(a.V), static_cast<float*>(a.O), a.L, a.N, q_tiles,
                     a.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, int d, hipStream_t stream) {
  if (d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace fa
