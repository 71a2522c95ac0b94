// Shared device helpers for the lattn HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lattn {

// bf16 values travel as raw 16-bit patterns; conversions are explicit.
using bf16_raw = uint16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_raw x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaN stays NaN, Inf stays Inf).
__device__ __forceinline__ bf16_raw f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) {
    return static_cast<bf16_raw>((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  }
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_raw>(u >> 16);
}

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};

template <>
struct Elem<bf16_raw> {
  static __device__ __forceinline__ float load(const bf16_raw* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(bf16_raw* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

}  // namespace lattn
