// Device-side helpers shared by the jt kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include "../../include/jt.h"

namespace jt {

constexpr int kWave = 64;
constexpr int kPage = 16;

__device__ __forceinline__ void report(int32_t* err, int bits) {
  if (err) atomicOr(err, bits);
}

// bf16 <-> f32 through bit patterns (exact widening; round-to-nearest-even
// narrowing).
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_bits_to_f32(p[i]);
}

// Total order on (value, id) used for top-W and argmax: larger value first,
// then smaller id.  Values are never NaN here (NaN inputs are rejected).
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ double shfl_xor_f64(double v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

}  // namespace jt
