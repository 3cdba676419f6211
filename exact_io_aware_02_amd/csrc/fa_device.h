// Device-side building blocks shared by the bf16 prefill kernels (forward
// and backward) on gfx950: vector types, buffer->LDS loads, the padded and
// permuted LDS row layout, lane-pair reductions and barriers.  Not part of
// the public ABI.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {
namespace dev {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

// Rows of a tile in LDS are padded by 16 bytes (stride 2d + 16), which makes
// the 16-byte row-fragment reads of the loops free of bank conflicts.  Tiles
// that are also read transposed (ds_read_b64_tr_b16) store their rows with
// the two 2-bit fields of (row mod 16) swapped, so the 4 consecutive rows of
// one transposing read land 4 stored rows apart; the map is an involution.
__host__ __device__ constexpr int vrow_perm(int k) {
  return (k & ~15) | ((k & 3) << 2) | ((k >> 2) & 3);
}

// Buffer resource (4 descriptor words) over `bytes` bytes at `base`, no
// stride.  A load whose offset is past the end returns zeros and touches no
// memory.  Whether a load's SGPR offset counts in that check differs between
// AMD GPU generations; gfx950 counts it, which the NaN-padded ragged-tail
// tests pin, so the C++ kernels put a tile's offset there.  (The generated
// d = 128 forward loop builds a resource per tile instead, at no cost.)
__device__ __forceinline__ u32x4_t make_rsrc(const void* base, unsigned bytes) {
  const unsigned long long a = (unsigned long long)base;
  return u32x4_t{(unsigned)a, (unsigned)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}
// 16 bytes per lane from rsrc[voff + soff] into LDS at lds + 16 * lane.
// Issued as asm so the compiler does not order it against LDS reads of other
// buffers (it cannot prove them disjoint and would drain the queue); every
// wait for these loads is explicit (vmcnt) in the kernels.  The compiler's
// hazard tracking does not look inside asm, so the leading s_nop 4 supplies
// the wait states a buffer load needs after a VALU write of one of its SGPR
// operands (v_readlane restoring a spilled descriptor: 5) and after the M0
// write that sets the LDS address (1).
__device__ __forceinline__ void load_lds16(u32x4_t rsrc, void LDS_AS* lds, unsigned voff, unsigned soff) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"((unsigned)(size_t)lds)
               : "memory");
}

// Offset, within a run of D-element bf16 rows in HBM, of the 16 bytes that
// belong at byte `o` of a padded LDS tile (rows permuted by vrow_perm when
// `permuted`); a padding slot gets an offset past any buffer end (reads as
// zero, touches no memory).
template <int D>
__device__ __forceinline__ unsigned padded_source(int o, bool permuted) {
  constexpr int kRowBytes = D * 2, kStride = kRowBytes + 16, kChunks = D / 8;
  const int p = o / kStride;
  const int ch = (o - p * kStride) >> 4;
  if (ch >= kChunks) return 0xFFFFFFF0u;
  const int row = permuted ? vrow_perm(p) : p;
  return (unsigned)(row * kRowBytes + ch * 16);
}

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, v);
}

// max / sum with lane l^32 (the other half of the same accumulator column);
// the swap returns (x[l & 31], x[32 + (l & 31)]) in every lane.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Marks x as used at this point, so its computation is not sunk past it.
// Input-only: the producing instruction stays the last writer of the
// registers, so the compiler still inserts the wait states its readers need.
// (The host pass parses kernel bodies too, and its target has no such
// register class for 64-byte operands, hence the guard.)
template <typename T>
__device__ __forceinline__ void keep(const T& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(x));
#endif
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// drain every load in flight): the caller waits for what must have landed.
// The empty asm statements keep the compiler from moving LDS accesses across.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// A transposing LDS read pair: 8 consecutive rows r0 + 8t + 4g + 0..3
// (t = 0, 1) of one 16-row step of a tile stored with vrow_perm, at column
// block `col_bytes`, as the A operand (rows on the k index) of a 32x32x16
// product; `base` is the per-lane address of the tile.
template <int kStride>
__device__ __forceinline__ bf16x8_t tr_frag(const char LDS_AS* base, int step, int col_bytes) {
  bf16x8_t a;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (i16x4_t LDS_AS*)(base + (step * 16 + 2 * t) * kStride + col_bytes));
    const bf16x4_t v4 = __builtin_bit_cast(bf16x4_t, v);
    a[4 * t + 0] = v4[0];
    a[4 * t + 1] = v4[1];
    a[4 * t + 2] = v4[2];
    a[4 * t + 3] = v4[3];
  }
  return a;
}

// Per-lane address offset, within a tile stored with vrow_perm, that
// tr_frag reads from: lanes address columns 16 ((lane >> 4) & 1) + 4 (lane & 3)
// of stored rows 4 ((lane & 15) >> 2) + g.
template <int kStride>
__device__ __forceinline__ int tr_lane_base(int lane) {
  const int g = lane >> 5;
  return (4 * ((lane & 15) >> 2) + g) * kStride + (((lane >> 4) & 1) * 16 + (lane & 3) * 4) * 2;
}

}  // namespace dev
}  // namespace fa
