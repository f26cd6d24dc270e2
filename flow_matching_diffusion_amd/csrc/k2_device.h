// Device-side building blocks shared by the gfx950 kernels of libk2.
//
// Matrix-core convention used by every kernel here: a 16x16 output tile is accumulated with
// mma16(acc, a, b), where each lane supplies an 8-element fragment of A and of B.
//   A fragment: lane l holds row (l % 16), k slots 8*(l/16) .. 8*(l/16)+7 of a 32-wide k chunk
//   B fragment: lane l holds column (l % 16), the same k slots
//   acc (4 floats): lane l holds column (l % 16), rows 4*(l/16) + r, r = 0..3
// For bf16 this is one v_mfma_f32_16x16x32_bf16. For fp32 it is eight v_mfma_f32_16x16x4_f32, the
// i-th taking element i of each lane's fragment. Since A and B always use the same (lane group,
// slot) -> k assignment, any permutation of k inside the chunk gives the same sum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace k2 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T> struct FragOf;
template <> struct FragOf<bf16> { typedef bf16x8 type; };
template <> struct FragOf<float> { typedef f32x8 type; };

__device__ __forceinline__ f32x4 mma16(f32x4 acc, const bf16x8& a, const bf16x8& b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma16(f32x4 acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
  return acc;
}

template <typename T> __device__ __forceinline__ T to_t(float x);
template <> __device__ __forceinline__ float to_t<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 to_t<bf16>(float x) { return (bf16)x; }  // RNE

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }

// Pack 8 floats into a fragment of T.
__device__ __forceinline__ void pack8(bf16x8& f, const float* v) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (bf16)v[i];
}
__device__ __forceinline__ void pack8(f32x8& f, const float* v) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = v[i];
}

// sigmoid(x) = 1 / (1 + e^-x) and silu(x) = x sigmoid(x), with the hardware reciprocal (v_rcp_f32,
// within 1 ulp) instead of a correctly rounded division, which compiles to a ten-instruction
// sequence: the SwiGLU epilogue takes 128 of them per lane and tile, the attention epilogue 64.
// Large negative x: e^-x overflows to inf and the reciprocal gives 0, as the division would.
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float siluf_(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float gelu_tanhf_(float x) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * x * (1.0f + tanhf(k0 * (x + 0.044715f * x * x * x)));
}

// Sum / max over the 16 lanes of a lane group (lanes with equal l/16).
__device__ __forceinline__ float group16_sum(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 8);
  return v;
}
// Over the 4 lane groups (lanes with equal l%16).
__device__ __forceinline__ float across_groups_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float across_groups_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Lanes of one wave passing data through LDS. The hardware runs a wave's LDS accesses in issue
// order, but the compiler reasons per lane: with nothing in between it may move or merge one lane's
// LDS read across another lane's write (it did: a staged epilogue re-used values read for the
// previous block). The wave-scope fences emit no instruction; they keep every LDS access on its side.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Buffer resources (raw, 32-bit offsets). A load whose offset lies past the resource's byte size
// returns zeros; kOOB is an offset past every resource, used to switch a lane's load off.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;

// LDS a workgroup may hold on gfx950 (static plus dynamic); a dispatch asking for more is rejected
// and aborts the queue, so every kernel checks its static LDS at compile time. wgs: workgroups the
// kernel's launch bounds expect to share one compute unit.
constexpr size_t kLdsBytes = 163840;
#define K2_LDS_CHECK(bytes, wgs) \
  static_assert((size_t)(bytes) * (wgs) <= kLdsBytes, "static LDS exceeds what the launch bounds allow")

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, size_t bytes) {
  const uint32_t n = bytes > 0x7FFFFFF0ull ? 0x7FFFFFF0u : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ uint4 bload(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// 16-byte store at byte offset off; dropped when off lies past the resource's byte size.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void bstore(rsrc_t r, uint32_t off, float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, 0);
}
__device__ __forceinline__ void bstore(rsrc_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, 0);
}

// 16-byte-per-lane DMA from a buffer into LDS at lds + 16 * lane (lds must be wave-uniform), from
// byte offset off (per lane) + soff (wave-uniform, scalar offset field). The builtin exists for the
// device pass only; the host pass (which only needs kernels' launch stubs) sees an empty body.
__device__ __forceinline__ void dma16(rsrc_t r, void* lds, uint32_t off, uint32_t soff = 0) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)off, (int)soff,
                                           0, 0);
#endif
}

// vmcnt(n) with expcnt and lgkmcnt left unconstrained, and lgkmcnt(0) alone (gfx9 s_waitcnt fields).
#define K2_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
#define K2_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

// XOR swizzle of 16-byte chunk positions within 128-byte LDS rows (8 chunks). Measured on gfx950
// with the LDS bank-conflict counter: ds_read_b128 of 16 consecutive rows x 4 consecutive chunks
// (the MFMA fragment pattern) and ds_write_b128 of 8 rows x 8 chunks both run conflict-free (4 LDS
// cycles per instruction, 256 bytes per cycle) with chunk ^ (row & 7); chunk ^ (row & 7) ^ (row >> 3 & 1)
// takes 8 cycles for the reads.
__device__ __forceinline__ int swz8(int row) { return row & 7; }

}  // namespace k2
