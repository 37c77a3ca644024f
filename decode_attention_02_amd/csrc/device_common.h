// Device helpers shared by the gfx950 kernels: bf16 <-> fp32 and element access.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace gqla {

typedef uint16_t bf16_t;  // bfloat16 bit pattern

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  return static_cast<bf16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

template <typename T> struct Elt;
template <> struct Elt<float> {
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elt<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

__device__ __forceinline__ void store_out(void* out, int32_t kind, int64_t i, float v) {
  if (kind == 0) static_cast<float*>(out)[i] = v;
  else static_cast<bf16_t*>(out)[i] = f32_to_bf16(v);
}

__device__ __forceinline__ float nan_f32() { return __uint_as_float(0x7fc00000u); }

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace gqla
