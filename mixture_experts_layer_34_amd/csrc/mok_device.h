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

// Unsigned 64-bit maximum over a wave through DPP lane moves (no LDS
// crossbar): swaps within quads, rotations by 4 and 8 within each row of 16
// lanes, then the broadcasts of lane 15 of each row to the next row and of
// lane 31 to rows 2 and 3; lane 63 ends with the maximum, which is returned
// to every lane.  A lane with no source in a step reads 0, the identity.
template <int CTRL>
__device__ __forceinline__ void dpp_max_step(uint32_t& hi, uint32_t& lo) {
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, CTRL, 0xf, 0xf, false);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, CTRL, 0xf, 0xf, false);
  const bool gt = ohi > hi || (ohi == hi && olo > lo);
  hi = gt ? ohi : hi;
  lo = gt ? olo : lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t key) {
  uint32_t hi = (uint32_t)(key >> 32), lo = (uint32_t)key;
  dpp_max_step<0xb1>(hi, lo);   // quad_perm [1,0,3,2]
  dpp_max_step<0x4e>(hi, lo);   // quad_perm [2,3,0,1]
  dpp_max_step<0x124>(hi, lo);  // row_ror 4
  dpp_max_step<0x128>(hi, lo);  // row_ror 8
  dpp_max_step<0x142>(hi, lo);  // row_bcast 15
  dpp_max_step<0x143>(hi, lo);  // row_bcast 31
  hi = (uint32_t)__builtin_amdgcn_readlane((int)hi, 63);
  lo = (uint32_t)__builtin_amdgcn_readlane((int)lo, 63);
  return ((uint64_t)hi << 32) | lo;
}

// ------------------------------------------------------------ status word
// Device-side checks report into the status word at the start of the
// workspace: word 0 becomes MOK_ERR_DEVICE (5) and word 1 gathers the bits of
// the checks that failed.  Each layer call clears both words first.
constexpr int32_t kStatusDevice = 5;                   // MOK_ERR_DEVICE
constexpr int32_t kCheckLogits = 1;                    // a router logit row holds NaN or +-Inf
constexpr int32_t kCheckIndex = 2;                     // a row or expert index outside its range
__device__ __forceinline__ void report(int32_t* status, int32_t bit) {
  if (status) {
    __hip_atomic_store(status, kStatusDevice, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_or(status + 1, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
// A row-map entry: -1 (remote slot) or a row in [0, rows).  Anything else is
// reported and read as -1, so no access ever leaves the row buffers.
__device__ __forceinline__ int32_t checked_row(int32_t r, int64_t rows, int32_t* status) {
  if (r < -1 || (int64_t)r >= rows) {
    report(status, kCheckIndex);
    return -1;
  }
  return r;
}

// SiLU and its derivative pieces in fp32.
__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

// OCP E4M3 (bias 7, no infinities) from an fp32 value: round to nearest even,
// saturate to +-448, keep the sign of zero.  The layer uses the gfx950
// conversion instruction on the value clamped to +-448 (e4m3_rne, e4m3x4);
// this software encoder, written from the format's definition, is the
// reference the diagnostic library checks that instruction against (equal on
// every float32 of magnitude below 512, both signs, subnormals included; the
// clamp makes the rest equal too).
__device__ __forceinline__ uint32_t e4m3_rne_sw(float v) {
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

__device__ __forceinline__ float e4m3_clamp(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const float c = e4m3_clamp(v);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
}
// Four codes packed little-endian: a | b << 8 | c << 16 | d << 24.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), w, true);
  return (uint32_t)w;
}

// Shared-scale exponent of an MX block from its amax (>= 0): floor(log2 amax) - 8,
// clamped to [-127, 127]; amax = 0 (or fp32-subnormal) gives -127.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  int ef = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  if (ef == 0) return -127;
  int s = ef - 127 - 8;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// OCP E2M1 (FP4: sign, two exponent bits with bias 1, one mantissa bit;
// magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) from an fp32 value: round to nearest
// even, saturate to +-6, keep the sign of zero.  The magnitude code is the
// number of rounding thresholds |v| reaches; at a midpoint the even code
// (mantissa bit 0) wins, i.e. the magnitude below for the midpoints 0.25,
// 1.25, 2.5 and 5, the one above for 0.75, 1.75 and 3.5.
__device__ __forceinline__ uint32_t e2m1_rne(float v) {
  const float a = fabsf(v);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(v) >> 28) & 8u);
}
// E2M1 codes of v[0..7] * 2^-se, element i in bits [4 i, 4 i + 4) (the byte
// order the scaled MFMA reads: the lower K element in the low nibble).
__device__ __forceinline__ uint32_t e2m1x8(const float* v, int se) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= e2m1_rne(ldexpf(v[i], -se)) << (4 * i);
  return w;
}

// Shared-scale exponent of an MXFP4 block: floor(log2 amax) - 2 (the largest
// E2M1 power of two is 2^2), clamped to [-127, 127]; amax = 0 (or
// fp32-subnormal) gives -127.
__device__ __forceinline__ int mx4_scale_exp(float amax) {
  int ef = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  if (ef == 0) return -127;
  int s = ef - 127 - 2;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// ------------------------------------------------------------ HBM -> LDS DMA
// Buffer resource (V#) of `bytes` bytes at p: stride 0, raw addressing;
// offsets at or past `bytes` read as zero.  All fields must be wave-uniform.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  return i32x4_t{(int32_t)(uint32_t)a, (int32_t)((uint32_t)(a >> 32) & 0xFFFFu), (int32_t)bytes, 0x00020000};
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One wave copies 64 x 16 bytes from the buffer (lane offset voff + soff) to
// LDS [lds, lds + 1024), lane i's bytes landing at lds + 16 i.  Written as
// inline assembly on purpose: the compiler cannot tell these LDS writes from
// the fragment reads of another pipeline stage, and would otherwise wait for
// every outstanding copy before each LDS read.  The caller owns the ordering:
// s_waitcnt vmcnt(n) (copies complete in issue order) and then a workgroup
// barrier before any wave reads what was copied.  `lds` must be wave-uniform;
// M0 is restored afterwards.
// With NT, the copy carries the non-temporal hint (the lines it brings into
// L2 are the first to be replaced).
template <bool NT = false>
__device__ __forceinline__ void dma_b128(i32x4_t rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  uint32_t save;
  if constexpr (NT) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen nt lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
        : "memory");
  }
}

// Like dma_b128 with 2 bytes per lane (any alignment): lane i's two bytes land
// zero-extended in the dword at lds + 4 i.
__device__ __forceinline__ void dma_u16(i32x4_t rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_ushort %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}
