// Diagnostic: one gfx950 scaled-MFMA block (v_mfma_scale_f32_32x32x64_f8f6f4,
// E4M3 operands, one E8M0 scale per 32 K values of each row) on caller-given
// codes and scales, so that a test can compare the matrix core's fp32 result
// with the exact sum of the same products.  Not part of the layer.
//
// Operand layout of the instruction as the layer's MXFP8 GEMMs feed it: lane
// l holds row l % 32 of its operand and the 16-byte pieces 16 h .. 16 h + 15
// and 32 + 16 h .. 32 + 16 h + 15 of that row's 64 K bytes (h = l / 32), and
// the scale of the row's K block h.  The result of lane l, register i, is
// C[(i / 4) * 8 + h * 4 + i % 4][l % 32].
#include "../../include/mok_diag.h"
#include "mok_device.h"

namespace {

__global__ __launch_bounds__(64) void mfma_scale_block_kernel(const uint8_t* __restrict__ a,
                                                              const uint8_t* __restrict__ b,
                                                              const uint8_t* __restrict__ sa,
                                                              const uint8_t* __restrict__ sb,
                                                              const float* __restrict__ c_in,
                                                              float* __restrict__ c_out) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int l = threadIdx.x, r = l & 31, h = l >> 5;
  typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 alo = *reinterpret_cast<const i32x4*>(a + r * 64 + 16 * h);
  const i32x4 ahi = *reinterpret_cast<const i32x4*>(a + r * 64 + 32 + 16 * h);
  const i32x4 blo = *reinterpret_cast<const i32x4*>(b + r * 64 + 16 * h);
  const i32x4 bhi = *reinterpret_cast<const i32x4*>(b + r * 64 + 32 + 16 * h);
  const i32x8_t av = __builtin_shufflevector(alo, ahi, 0, 1, 2, 3, 4, 5, 6, 7);
  const i32x8_t bv = __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7);
  const int sa_l = sa[r * 2 + h], sb_l = sb[r * 2 + h];
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = c_in[((i >> 2) * 8 + h * 4 + (i & 3)) * 32 + r];
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, sa_l, 0, sb_l);
#pragma unroll
  for (int i = 0; i < 16; ++i) c_out[((i >> 2) * 8 + h * 4 + (i & 3)) * 32 + r] = acc[i];
#endif
}

}  // namespace

extern "C" int32_t mok_diag_mfma_scale_block(const uint8_t* a, const uint8_t* b, const uint8_t* sa,
                                             const uint8_t* sb, const float* c_in, float* c_out, void* stream) {
  if (!a || !b || !sa || !sb || !c_in || !c_out) return 1;
  hipLaunchKernelGGL(mfma_scale_block_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, a, b, sa, sb, c_in, c_out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
