// Device-side helpers shared by the MoE layer kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bf16 storage
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define MOK_WAVE 64

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f2bf(v); }

// Butterfly reductions over the 64 lanes of a wave; every lane gets the result
// and the combination order is fixed, so the result is run-to-run identical.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// SiLU and its derivative pieces in fp32.
__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

// OCP E4M3 (bias 7, no infinities) from an fp32 value: round to nearest even,
// saturate to +-448, keep the sign of zero.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fminf(fabsf(v), 448.0f);
  uint32_t au = __float_as_uint(a);
  int e = (int)(au >> 23) - 127;
  uint32_t code;
  if (e < -6) {
    // spacing 2^-9 below the smallest normal; n = 8 is the code of 2^-6
    code = (uint32_t)rintf(a * 512.0f);
  } else {
    uint32_t r = au + 0x7FFFFu + ((au >> 20) & 1u);  // keep 3 fraction bits, RNE
    int e2 = (int)(r >> 23) - 127;
    code = ((uint32_t)(e2 + 7) << 3) | ((r >> 20) & 7u);
  }
  return sign | code;
}

// Shared-scale exponent of an MX block from its amax (>= 0): floor(log2 amax) - 8,
// clamped to [-127, 127]; amax = 0 (or fp32-subnormal) gives -127.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  int ef = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  if (ef == 0) return -127;
  int s = ef - 127 - 8;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}
