// Two measurement kernels that give the roofline its measured ceilings next
// to the published peaks: a read-only HBM stream and a loop of bf16 MFMAs.
// They compute nothing of attention; the benchmark times them in the same
// process as the attention kernels.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Every thread reads 16-byte words i = gid, gid + stride, ... < n16, eight
// independent non-temporal loads in flight per step (of the variants timed,
// 4, 8 or 16 loads per step, temporal or not, 2 to 256 workgroups per
// compute unit, this one with 64 workgroups per compute unit read fastest).
// The loaded words are folded into one integer that is stored only if it
// equals a value no input of the benchmark produces, so the kernel writes
// (almost) nothing while the loads cannot be dropped.  Every access is below
// n16 words by construction.
__global__ __launch_bounds__(256) void probe_hbm_read_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                              uint32_t* __restrict__ sink) {
  constexpr int kU = 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kU - 1) * stride < n16; i += kU * stride) {
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
    uint32_t s = 0;
#pragma unroll
    for (int u = 0; u < kU; ++u) s += v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    acc ^= s;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(buf + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

// Each wavefront runs `iters` rounds of four independent
// v_mfma_f32_32x32x16_bf16 chains (4 x 32768 FLOP per round).  Wavefront 0
// of a workgroup records the shader-clock cycles (s_memtime) and the 100 MHz
// constant-clock ticks (s_memrealtime) it spent, from which the host derives
// the clock the loop ran at.  Every thread stores one float of its
// accumulators, so the products cannot be dropped.
__global__ __launch_bounds__(256) void probe_mfma_bf16_kernel(int iters, float* __restrict__ sink,
                                                               uint64_t* __restrict__ stamps) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)(0.001f * (float)((lane + k) & 7));
    b[k] = (__bf16)(0.002f * (float)((lane * 3 + k) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int k = 0; k < 16; ++k) s += c0[k] + c1[k] + c2[k] + c3[k];
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0 && stamps) {
    stamps[2 * blockIdx.x] = t1 - t0;
    stamps[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// The same loop with operands that change from one product to the next,
// like the attention kernels' fragments: each of the four chains has its own
// A and B, filled from an integer hash of (seed, workgroup, lane, chain,
// element) with values in [-2, 2), and the chains take turns.  The loop
// above multiplies small multiples of 0.001 and 0.002, many of them zero;
// with random bf16 values held constant it runs within 4 % of this one, so
// the operand values, more than their changing between products, set the
// power the products draw and so the clock.
__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(256) void probe_mfma_bf16_mixed_kernel(int iters, uint32_t seed, float* __restrict__ sink,
                                                                     uint64_t* __restrict__ stamps) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[4], b[4];
  for (int c = 0; c < 4; ++c)
    for (int k = 0; k < 8; ++k) {
      const uint32_t base = seed * 0x9e3779b9u ^ ((blockIdx.x * 256 + threadIdx.x) * 64 + c * 16 + k);
      a[c][k] = (__bf16)((float)(probe_hash(2 * base) >> 8) * 0x1p-22f - 2.f);
      b[c][k] = (__bf16)((float)(probe_hash(2 * base + 1) >> 8) * 0x1p-22f - 2.f);
    }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[2], c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], b[3], c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int k = 0; k < 16; ++k) s += c0[k] + c1[k] + c2[k] + c3[k];
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0 && stamps) {
    stamps[2 * blockIdx.x] = t1 - t0;
    stamps[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

hipError_t launch_probe_mfma_bf16_mixed(int workgroups, int iters, uint32_t seed, float* sink, uint64_t* stamps,
                                        hipStream_t stream) {
  hipLaunchKernelGGL(probe_mfma_bf16_mixed_kernel, dim3(workgroups), dim3(256), 0, stream, iters, seed, sink, stamps);
  return hipGetLastError();
}

hipError_t launch_probe_hbm_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(probe_hbm_read_kernel, dim3(workgroups), dim3(256), 0, stream,
                     static_cast<const u32x4*>(buf), (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

hipError_t launch_probe_mfma_bf16(int workgroups, int iters, float* sink, uint64_t* stamps, hipStream_t stream) {
  hipLaunchKernelGGL(probe_mfma_bf16_kernel, dim3(workgroups), dim3(256), 0, stream, iters, sink, stamps);
  return hipGetLastError();
}

}  // namespace fa
