// Device-side helpers shared by the KLA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kla {

constexpr int kWave = 64;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- element conversion -------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename E>
__device__ __forceinline__ E from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }  // RNE

// 16-byte vector of E: 8 bf16 or 4 float.
template <typename E>
struct Vec16;
template <>
struct Vec16<bf16> {
  static constexpr int N = 8;
  typedef bf16x8 type;
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  typedef f32x4 type;
};

// ---- wave reductions / scans ----------------------------------------------------------
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// Sum over groups of G consecutive lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    float y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

}  // namespace kla
