// Diagnostics of the gfx950 instructions the MXFP8 and MXFP4 paths rely on.  One
// scaled-MFMA block (v_mfma_scale_f32_32x32x64_f8f6f4,
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

// The same instruction on caller-given operand registers: lane l's eight A
// and eight B dwords, its two scale bytes and its sixteen accumulators, for
// operand formats FA (A) and FB (B) (0 E4M3, 4 E2M1: then only the first four
// dwords are read), so that a test can establish how the instruction maps
// register bits to K for a format.
template <int FA, int FB>
__global__ __launch_bounds__(64) void mfma_scale_raw_kernel(const uint32_t* __restrict__ a,
                                                            const uint32_t* __restrict__ b,
                                                            const uint8_t* __restrict__ sa,
                                                            const uint8_t* __restrict__ sb,
                                                            const float* __restrict__ c_in,
                                                            float* __restrict__ c_out) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int l = threadIdx.x;
  i32x8_t av, bv;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    av[i] = (int32_t)a[l * 8 + i];
    bv[i] = (int32_t)b[l * 8 + i];
  }
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = c_in[l * 16 + i];
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, FA, FB, 0, (int)sa[l], 0, (int)sb[l]);
#pragma unroll
  for (int i = 0; i < 16; ++i) c_out[l * 16 + i] = acc[i];
#endif
}

// Every float32 of magnitude below 2^9 (bit patterns [0, n), both signs)
// through the layer's E4M3 encoders: the conversion instruction (e4m3_rne,
// and e4m3x4 with the value in each of its four byte places) against the
// software encoder of the format's definition.  Per thread: mismatches and
// the first mismatching bit pattern (0xFFFFFFFF: none).
__global__ __launch_bounds__(256) void e4m3_check_kernel(uint32_t n, uint32_t* __restrict__ count,
                                                         uint32_t* __restrict__ first) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t tid = blockIdx.x * 256 + threadIdx.x, stride = gridDim.x * 256;
  uint32_t cnt = 0, f = 0xFFFFFFFFu;
  for (uint32_t u = tid; u < n; u += stride)
    for (int sgn = 0; sgn < 2; ++sgn) {
      const uint32_t bits = u | (sgn ? 0x80000000u : 0u);
      const float x = __uint_as_float(bits);
      const uint32_t sw = e4m3_rne_sw(x);
      const uint32_t q = (u >> 7) & 3u;  // the byte place this value takes in e4m3x4
      const uint32_t w = e4m3x4(q == 0 ? x : 1.0f, q == 1 ? x : 1.0f, q == 2 ? x : 1.0f, q == 3 ? x : 1.0f);
      const uint32_t one = 0x38u;  // E4M3 code of 1.0
      uint32_t expect = 0;
      for (uint32_t i = 0; i < 4; ++i) expect |= (i == q ? sw : one) << (8 * i);
      if (e4m3_rne(x) != sw || w != expect) {
        ++cnt;
        if (f == 0xFFFFFFFFu) f = bits;
      }
    }
  count[tid] = cnt;
  first[tid] = f;
#endif
}

}  // namespace

extern "C" int32_t mok_diag_e4m3_check(uint32_t n, uint32_t* count, uint32_t* first, int32_t blocks, void* stream) {
  if (!count || !first || blocks < 1 || n > 0x44000000u) return 1;
  hipLaunchKernelGGL(e4m3_check_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, n, count, first);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int32_t mok_diag_mfma_scale_raw(const uint32_t* a, const uint32_t* b, const uint8_t* sa,
                                           const uint8_t* sb, const float* c_in, float* c_out, int32_t fmt_a,
                                           int32_t fmt_b, void* stream) {
  if (!a || !b || !sa || !sb || !c_in || !c_out) return 1;
  const hipStream_t s = (hipStream_t)stream;
  if (fmt_a == 0 && fmt_b == 0)
    hipLaunchKernelGGL((mfma_scale_raw_kernel<0, 0>), dim3(1), dim3(64), 0, s, a, b, sa, sb, c_in, c_out);
  else if (fmt_a == 4 && fmt_b == 4)
    hipLaunchKernelGGL((mfma_scale_raw_kernel<4, 4>), dim3(1), dim3(64), 0, s, a, b, sa, sb, c_in, c_out);
  else if (fmt_a == 4 && fmt_b == 0)
    hipLaunchKernelGGL((mfma_scale_raw_kernel<4, 0>), dim3(1), dim3(64), 0, s, a, b, sa, sb, c_in, c_out);
  else
    return 1;
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int32_t mok_diag_mfma_scale_block(const uint8_t* a, const uint8_t* b, const uint8_t* sa,
                                             const uint8_t* sb, const float* c_in, float* c_out, void* stream) {
  if (!a || !b || !sa || !sb || !c_in || !c_out) return 1;
  hipLaunchKernelGGL(mfma_scale_block_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, a, b, sa, sb, c_in, c_out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
