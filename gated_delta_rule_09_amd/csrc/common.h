// common.h -- device helpers shared by the gfx950 kernels of libgdn.
//
// Storage formats, 64-lane wave reductions and the MFMA operand conventions
// used by the prefill kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bfloat16

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Unpack 8 bf16 held in a 16-byte vector.
__device__ __forceinline__ void bf16x8_to_f32(const uint4 p, float* f) {
  f[0] = __uint_as_float(p.x << 16);
  f[1] = __uint_as_float(p.x & 0xffff0000u);
  f[2] = __uint_as_float(p.y << 16);
  f[3] = __uint_as_float(p.y & 0xffff0000u);
  f[4] = __uint_as_float(p.z << 16);
  f[5] = __uint_as_float(p.z & 0xffff0000u);
  f[6] = __uint_as_float(p.w << 16);
  f[7] = __uint_as_float(p.w & 0xffff0000u);
}

__device__ __forceinline__ uint4 f32_to_bf16x8(const float* f) {
  uint4 p;
  p.x = static_cast<uint32_t>(f32_to_bf16(f[0])) | (static_cast<uint32_t>(f32_to_bf16(f[1])) << 16);
  p.y = static_cast<uint32_t>(f32_to_bf16(f[2])) | (static_cast<uint32_t>(f32_to_bf16(f[3])) << 16);
  p.z = static_cast<uint32_t>(f32_to_bf16(f[4])) | (static_cast<uint32_t>(f32_to_bf16(f[5])) << 16);
  p.w = static_cast<uint32_t>(f32_to_bf16(f[6])) | (static_cast<uint32_t>(f32_to_bf16(f[7])) << 16);
  return p;
}

// ---------------------------------------------------------------- reductions
//
// DPP sums inside groups of 8 and 16 lanes of a 64-lane wave.  After the call
// every lane of the group holds the group total.

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

// quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141,
// row_mirror = 0x140.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  return x;
}

__device__ __forceinline__ float sum16(float x) {
  x = sum8(x);
  x += dpp<0x140>(x);
  return x;
}

// ---------------------------------------------------------------- MFMA
//
// v_mfma_f32_16x16x32_f16: D[16x16] += A[16x32] * B[32x16].
//   A: lane l holds row (l % 16), 8 values of one lane group g = l / 16.
//   B: lane l holds column (l % 16), 8 values of lane group g.
//   C/D: lane l holds column (l % 16), rows 4g .. 4g+3.
// The hardware pairs element e of A in lane (row, g) with element e of B in
// lane (col, g); which reduction index a (g, e) slot stands for is a free
// choice as long as A and B agree.  The kernels use
//     kappa(g, e) = (e < 4) ? 4g + e : 16 + 4g + (e - 4)
// inside each block of 32 reduction indices, because then the accumulator of
// two vertically adjacent 16x16 tiles (rows 4g+e of tile 0, then of tile 1) is
// already a B operand for a reduction over those 32 rows: no LDS round trip.
// v_mfma_f32_16x16x16_f16 uses kappa(g, e) = 4g + e, which is the accumulator
// layout of one tile.

__device__ __forceinline__ floatx4 mfma32(const half8 a, const half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma16(const half4 a, const half4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half4 to_half4(const floatx4 x) {
  half4 h;
  h[0] = static_cast<_Float16>(x[0]);
  h[1] = static_cast<_Float16>(x[1]);
  h[2] = static_cast<_Float16>(x[2]);
  h[3] = static_cast<_Float16>(x[3]);
  return h;
}

// Two stacked accumulator tiles -> one B operand over their 32 rows.
__device__ __forceinline__ half8 to_half8(const floatx4 lo, const floatx4 hi) {
  half8 h;
  h[0] = static_cast<_Float16>(lo[0]);
  h[1] = static_cast<_Float16>(lo[1]);
  h[2] = static_cast<_Float16>(lo[2]);
  h[3] = static_cast<_Float16>(lo[3]);
  h[4] = static_cast<_Float16>(hi[0]);
  h[5] = static_cast<_Float16>(hi[1]);
  h[6] = static_cast<_Float16>(hi[2]);
  h[7] = static_cast<_Float16>(hi[3]);
  return h;
}

__device__ __forceinline__ half8 cat8(const half4 lo, const half4 hi) {
  half8 h;
  h[0] = lo[0]; h[1] = lo[1]; h[2] = lo[2]; h[3] = lo[3];
  h[4] = hi[0]; h[5] = hi[1]; h[6] = hi[2]; h[7] = hi[3];
  return h;
}

// Work-group barrier that orders LDS only: each wave waits for its own LDS
// operations, then all waves meet.  Unlike __syncthreads() it does not wait for
// global loads or stores in flight, so loads issued ahead (prefetch of the next
// chunk) stay in flight across it.  Use only where the barrier guards LDS.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Asynchronous copy of 16 bytes per lane from global memory straight into LDS
// (gfx950 global_load_lds_dwordx4): lane l's bytes land at lds_wave_base + 16 l,
// where lds_wave_base must be the same for the whole wave.  Completion is
// tracked by vmcnt only; wait with dma_barrier() before reading the data.
typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((global_void*)(src), (lds_void*)(lds_wave_base), 16, 0, 0);
}

// Work-group barrier after all of this wave's vector memory operations (loads,
// stores and LDS copies) and LDS operations have completed.
__device__ __forceinline__ void dma_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

constexpr int kWave = 64;

}  // namespace gdn
