// Internal helpers of libfa3q (device helpers for gfx950 and host-side validation).
// Not part of the public ABI; the public declarations live in include/fa3q.h.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>

#include "fa3q.h"

namespace fa3q {

constexpr int kWave = 64;

// ---------------------------------------------------------------- host helpers

inline bool is_aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Status after one or more kernel launches on the calling thread.
inline int launch_status() {
  return hipGetLastError() == hipSuccess ? FA3Q_OK : FA3Q_ERR_HIP;
}

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Number of compute units of the current device (cached per device id).
int device_cu_count();

// LDS bytes one workgroup may use on the current device (cached per device id).
int device_max_lds_per_block();

// Raise a kernel's dynamic-LDS limit once per process when it needs more than 64 KiB.
int allow_dynamic_lds(const void* kernel, size_t bytes);

constexpr size_t kLdsLimit = 160 * 1024;  // LDS per workgroup on gfx950

// ---------------------------------------------------------------- device helpers

// bf16 pair in one dword -> float32 of the low / high element (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float16 pair in one dword -> float32 of the low / high element (exact widening).
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// The low / high element of a pair of 16-bit floats: float16 when kF16, else bf16.
template <bool kF16>
__device__ __forceinline__ float lo16(uint32_t w) {
  if constexpr (kF16) return f16_lo(w);
  else return bf16_lo(w);
}
template <bool kF16>
__device__ __forceinline__ float hi16(uint32_t w) {
  if constexpr (kF16) return f16_hi(w);
  else return bf16_hi(w);
}

// Workgroup barrier that orders LDS traffic only (no wait on outstanding global loads).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

// Data-parallel-primitive move of a float inside a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G consecutive lanes; every lane of a group gets the sum.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (G >= 4) v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (G >= 8) v += dpp_f32<0x141>(v);  // row_half_mirror: pairs the two quads of 8 lanes
  if constexpr (G >= 16) v += dpp_f32<0x140>(v); // row_mirror: pairs the two halves of a 16-lane row
  if constexpr (G >= 32) v += __shfl_xor(v, 16);
  if constexpr (G >= 64) v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace fa3q
