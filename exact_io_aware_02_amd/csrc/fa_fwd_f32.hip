// FlashAttention forward for fp32 Q/K/V on gfx950, every step in fp32.
//
// Algorithm 1 of "Infra: Flash Attention" (section "Tiled computation and
// forward") with B_r = B_c = 64: a workgroup is one wavefront that owns 64
// query rows, one row per lane; K_j and V_j tiles of 64 keys are staged in
// LDS (read by every lane at the same address, i.e. broadcast), and each
// lane keeps its row's (m, l, u) state in registers.  The scores of a tile
// are formed, a row whose keys are all masked in this tile skips the update
// ("Notation and boundary conditions"), otherwise m' = max(m, rowmax S),
// alpha = e^{(m - m') scale}, W = e^{(S - m') scale}, l = alpha l + sum W,
// u = alpha u + W V_j.  At the end O = u / l and L = m*scale + ln l.
//
// This path exists for an fp32-input workload that is checked to 1e-5; it is
// tiny (a handful of workgroups), so it uses plain VALU FMAs rather than the
// reduced-precision matrix path of the bf16 kernel.

#include "fa_internal.h"

namespace fa {
namespace {

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void fwd_f32_kernel(const float* __restrict__ Qg,
                                                     const float* __restrict__ Kg,
                                                     const float* __restrict__ Vg,
                                                     float* __restrict__ Og, float* __restrict__ Lg,
                                                     int N, int q_tiles, float scale) {
  __shared__ __attribute__((aligned(16))) float Ks[kF32BC][D];
  __shared__ __attribute__((aligned(16))) float Vs[kF32BC][D];

  const int lane = threadIdx.x;
  const int bh = blockIdx.x / q_tiles;
  const int qt = blockIdx.x - bh * q_tiles;
  const size_t head_off = (size_t)bh * N * D;
  const int qrow = qt * kF32BR + lane;

  float q[D];
#pragma unroll
  for (int e = 0; e < D; e += 4) {
    float4 v = (qrow < N) ? *reinterpret_cast<const float4*>(Qg + head_off + (size_t)qrow * D + e)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    q[e] = v.x; q[e + 1] = v.y; q[e + 2] = v.z; q[e + 3] = v.w;
  }

  int n_tiles = (N + kF32BC - 1) / kF32BC;
  if (CAUSAL) {
    int last = qt * kF32BR + kF32BR - 1;
    if (last > N - 1) last = N - 1;
    n_tiles = min(n_tiles, last / kF32BC + 1);
  }

  float m = -INFINITY, l = 0.f;
  float u[D];
#pragma unroll
  for (int e = 0; e < D; ++e) u[e] = 0.f;

  for (int j = 0; j < n_tiles; ++j) {
    const int kbase = j * kF32BC;
    __syncthreads();  // previous tile fully consumed
    for (int idx = lane; idx < kF32BC * D / 4; idx += 64) {
      const int r = idx / (D / 4), c4 = (idx % (D / 4)) * 4;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (kbase + r < N) {
        kv = *reinterpret_cast<const float4*>(Kg + head_off + (size_t)(kbase + r) * D + c4);
        vv = *reinterpret_cast<const float4*>(Vg + head_off + (size_t)(kbase + r) * D + c4);
      }
      *reinterpret_cast<float4*>(&Ks[r][c4]) = kv;
      *reinterpret_cast<float4*>(&Vs[r][c4]) = vv;
    }
    __syncthreads();

    float s[kF32BC];
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kF32BC; ++k) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < D; e += 4) {
        float4 kv = *reinterpret_cast<const float4*>(&Ks[k][e]);
        acc = fmaf(q[e], kv.x, acc);
        acc = fmaf(q[e + 1], kv.y, acc);
        acc = fmaf(q[e + 2], kv.z, acc);
        acc = fmaf(q[e + 3], kv.w, acc);
      }
      const int key = kbase + k;
      const bool valid = key < N && (!CAUSAL || key <= qrow);
      s[k] = valid ? acc : -INFINITY;
      mx = fmaxf(mx, s[k]);
    }
    if (mx == -INFINITY) continue;  // every key of this tile masked for this row

    const float m_new = fmaxf(m, mx);
    const float alpha = (m == -INFINITY) ? 0.f : expf((m - m_new) * scale);
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) u[e] *= alpha;
#pragma unroll
    for (int k = 0; k < kF32BC; ++k) {
      const float p = expf((s[k] - m_new) * scale);  // exp(-inf) = 0 for masked keys
      rs += p;
#pragma unroll
      for (int e = 0; e < D; e += 4) {
        float4 vv = *reinterpret_cast<const float4*>(&Vs[k][e]);
        u[e] = fmaf(p, vv.x, u[e]);
        u[e + 1] = fmaf(p, vv.y, u[e + 1]);
        u[e + 2] = fmaf(p, vv.z, u[e + 2]);
        u[e + 3] = fmaf(p, vv.w, u[e + 3]);
      }
    }
    l = alpha * l + rs;
    m = m_new;
  }

  if (qrow < N) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int e = 0; e < D; e += 4) {
      *reinterpret_cast<float4*>(Og + head_off + (size_t)qrow * D + e) =
          make_float4(u[e] * inv, u[e + 1] * inv, u[e + 2] * inv, u[e + 3] * inv);
    }
    if (Lg != nullptr) Lg[(size_t)bh * N + qrow] = l > 0.f ? m * scale + logf(l) : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int q_tiles = (a.N + kF32BR - 1) / kF32BR;
  const int64_t nb = (int64_t)a.B * a.H * q_tiles;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)nb), dim3(64), 0, stream,
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
