// csa2_device.h -- device helpers shared by the CSA2 HIP kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa2.h"

namespace csa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// The hipError_t behind the most recent csa2_* call of the calling thread: one
// slot per thread (defined in api.hip); every entry point clears it on entry
// and sets it when a launch fails.
__attribute__((visibility("hidden"))) void set_last_hip_error(int e);

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Order-preserving map float -> uint32 (larger float -> larger key); -0 -> +0.
__device__ __forceinline__ uint32_t sortable(float f) {
  uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unsortable(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// E4M3 (OCP FN) byte -> float; exact. Codes 0x7F/0xFF (NaN) never occur in
// records written by csa2_quant_append.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (b & 0x80u) ? -mag : mag;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    T x = __shfl_xor(v, o, kWave);
    v = x > v ? x : v;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, kWave));
  return v;
}

// Work-group barrier that orders LDS only: unlike __syncthreads it does not
// wait for the thread's global loads in flight, which keep overlapping the
// steps after the barrier.  For code whose threads exchange data through LDS
// alone.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Cross-lane steps through DPP (row-local moves and row broadcasts of the
// gfx9 wave), which stay in the vector ALU instead of the LDS crossbar that
// shuffles use.  dpp0 reads 0 where a lane has no source.
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ uint32_t dpp0(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWMASK, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  x += dpp0<0x111>(x);        // row_shr:1
  x += dpp0<0x112>(x);        // row_shr:2
  x += dpp0<0x114>(x);        // row_shr:4
  x += dpp0<0x118>(x);        // row_shr:8
  x += dpp0<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
  x += dpp0<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}

// Wave-wide reductions (result in every lane): within each row of 16 lanes
// by quad and mirror moves, then across the four rows by readlane.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, dpp0<0xB1>(v));    // quad_perm [1,0,3,2]
  v = op(v, dpp0<0x4E>(v));    // quad_perm [2,3,0,1]
  v = op(v, dpp0<0x141>(v));   // row_half_mirror
  v = op(v, dpp0<0x140>(v));   // row_mirror
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return op(op(a, b), op(c, d));
}
__device__ __forceinline__ uint32_t wave_min_dpp(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
}
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
}
__device__ __forceinline__ uint32_t wave_sum_dpp(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t x, uint32_t y) { return x + y; });
}

// Agent-scope acquire/release counter used by the "last work-group of a
// problem finishes the job" pattern.
__device__ __forceinline__ uint32_t atomic_inc_acq_rel(uint32_t* p) {
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace csa2
