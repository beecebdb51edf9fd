// Data-movement steps of the layer: dispatch (gather tokens into the
// expert-contiguous buffer, optionally quantising to MXFP8), combine (the
// gate-weighted sum back in token order), and the reverse-combine of the
// backward pass with the router gradient.
//
// Dispatch sends every token to its experts and combine brings each result
// back to the token's place (kucoin.com, "Cursor's MoK réalise une
// amélioration des performances de 2,37x sur NVIDIA GB300 NVL72", section 01);
// the benchmarked layer ends with the final weighted sum (section 03); MXFP8
// activation quantisation is fused into the dispatch path instead of a
// separate kernel and HBM round trip (section 02).  The pages state that the
// layer is deterministic (laura-martel.com post on Mixture-of-Kittens, section
// "Le déterminisme est la partie sous-estimée"): every sum here runs in a fixed
// order (slot j ascending, then a fixed reduction tree), with no float atomics.
//
// All kernels are bound by HBM: each token row is read once and its k
// destination rows are written with 16-byte coalesced accesses.
#include "mok_device.h"
#include "mok_internal.h"

namespace mok {

constexpr int kMaxK = 1024;

// A row seen through a buffer resource: `row_bytes` bytes for a local slot
// (r >= 0), none for a remote one (r = -1), whose loads then return zeros and
// whose stores are dropped, without a branch or a memory access.  The index
// is the same for every lane, so the resource sits in scalar registers.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t row_rsrc(const void* base, int32_t r, int row_bytes) {
  const char* p = (const char*)base + (r >= 0 ? (int64_t)r * row_bytes : 0);
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, r >= 0 ? row_bytes : 0, 0x00020000);
}
// The rows gathered by the combine and the reverse-combine are read once per
// call, so those loads carry the non-temporal hint (cache policy bit 1): the
// combine went from 118 to 106 us at T 8192, d 4096, k 8 (5.7 TB/s).  On the
// stores the same hint was faster in isolation (a dispatch, 117 to 103 us)
// but slower inside the layer (the regather 117 to 141 us, the reverse-
// combine 219 to 230 us), so stores keep the default policy.
constexpr int kNT = 2;
__device__ __forceinline__ uint4 buf_load16(rsrc_t rs, int off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNT);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void buf_store16(rsrc_t rs, int off, uint4 u) {
  __builtin_amdgcn_raw_buffer_store_b128(decltype(__builtin_amdgcn_raw_buffer_load_b128(rs, 0, 0, 0)){u.x, u.y, u.z, u.w},
                                         rs, off, 0, 0);
}

__device__ __forceinline__ void buf_store8(rsrc_t rs, int off, uint2 u) {
  __builtin_amdgcn_raw_buffer_store_b64(decltype(__builtin_amdgcn_raw_buffer_load_b64(rs, 0, 0, 0)){u.x, u.y}, rs, off,
                                        0, 0);
}

// ------------------------------------------------------------------ dispatch
// One block per token: read x[t] once (16-byte vectors), write it to the
// rows of its local pairs.  The token's row indices are the same for every
// lane (scalar loads, no block barrier); they are taken in groups of eight,
// x[t] being re-read (from cache) per group when k > 8.  Each destination row
// is a buffer resource of size 0 for a remote slot, whose stores are dropped.
constexpr int kSlotGroup = 8;

template <typename T>
__global__ __launch_bounds__(256) void dispatch_gather_kernel(const T* __restrict__ x,
                                                              const int32_t* __restrict__ rop, int ntok,
                                                              int k, int d, T* __restrict__ xp, int64_t xp_rows,
                                                              int32_t* __restrict__ status) {
  const int nv = d * (int)sizeof(T) / 16;
  for (int t = blockIdx.x; t < ntok; t += gridDim.x) {
    const int32_t* tr = rop + (int64_t)t * k;
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)t * d);
    for (int j0 = 0; j0 < k; j0 += kSlotGroup) {
      rsrc_t rs[kSlotGroup];
      int32_t rv_[kSlotGroup];
#pragma unroll
      for (int i = 0; i < kSlotGroup; ++i) {
        const int jc = j0 + i < k ? j0 + i : k - 1;
        const int32_t rv = checked_row(tr[jc], xp_rows, status);
        rv_[i] = (j0 + i < k) ? rv : -1;
        rs[i] = row_rsrc(xp, rv_[i], d * (int)sizeof(T));
      }
      for (int v = threadIdx.x; v < nv; v += 256) {
        const uint4 val = src[v];
#pragma unroll
        for (int i = 0; i < kSlotGroup; ++i)
          if (rv_[i] >= 0) buf_store16(rs[i], 16 * v, val);
      }
    }
  }
}

hipError_t launch_dispatch_gather(const void* x, const int32_t* row_of_pair, int T, int k, int d, int bf16,
                                  void* xp, int64_t xp_rows, int32_t* status, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int blocks = T < 16384 ? T : 16384;
  if (bf16)
    hipLaunchKernelGGL(dispatch_gather_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s,
                       (const bf16_t*)x, row_of_pair, T, k, d, (bf16_t*)xp, xp_rows, status);
  else
    hipLaunchKernelGGL(dispatch_gather_kernel<float>, dim3(blocks), dim3(256), 0, s, (const float*)x,
                       row_of_pair, T, k, d, (float*)xp, xp_rows, status);
  return hipGetLastError();
}

// MX quantisation of 8 consecutive bf16 values held by one lane; four
// consecutive lanes form one block of 32.  Writes 8 E4M3 codes and, from the
// first lane of the group, the E8M0 scale byte.
__device__ __forceinline__ void mx_quant8(const uint4 v, uint2& codes, uint8_t& scale_byte) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const int se = mx_scale_exp(amax);
  codes.x = e4m3x4(ldexpf(f[0], -se), ldexpf(f[1], -se), ldexpf(f[2], -se), ldexpf(f[3], -se));
  codes.y = e4m3x4(ldexpf(f[4], -se), ldexpf(f[5], -se), ldexpf(f[6], -se), ldexpf(f[7], -se));
  scale_byte = (uint8_t)(se + 127);
}

// One block per token, 16 elements per lane: two lanes hold one MX block of
// 32, four lanes the two blocks of one 64-wide K step, whose scale bytes are
// adjacent in the pair-plane layout and go out as one 2-byte store.  Codes go
// out as 16-byte stores through per-row buffer resources (size 0, stores
// dropped, for remote slots).  d % 64 == 0, so a group of four lanes is
// active or inactive as a whole.
__global__ __launch_bounds__(256) void dispatch_gather_mxfp8_kernel(const bf16_t* __restrict__ x,
                                                                    const int32_t* __restrict__ rop, int ntok,
                                                                    int k, int d, uint8_t* __restrict__ xq,
                                                                    uint8_t* __restrict__ xs, int64_t xs_rows,
                                                                    int32_t* __restrict__ status) {
  const int nv = d / 16;
  const int lane = lane_id();
  for (int t = blockIdx.x; t < ntok; t += gridDim.x) {
    const int32_t* tr = rop + (int64_t)t * k;
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)t * d);
    for (int j0 = 0; j0 < k; j0 += kSlotGroup) {
      int32_t r[kSlotGroup];
      rsrc_t rs[kSlotGroup];
#pragma unroll
      for (int i = 0; i < kSlotGroup; ++i) {
        const int jc = j0 + i < k ? j0 + i : k - 1;
        const int32_t rv = checked_row(tr[jc], xs_rows, status);
        r[i] = (j0 + i < k) ? rv : -1;
        rs[i] = row_rsrc(xq, r[i], d);
      }
      for (int v = threadIdx.x; v < nv; v += 256) {
        const uint4 w0 = src[2 * v], w1 = src[2 * v + 1];
        const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        float f[16];
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          f[2 * i] = __uint_as_float(w[i] << 16);
          f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
          amax = fmaxf(amax, fmaxf(fabsf(f[2 * i]), fabsf(f[2 * i + 1])));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
        const int se = mx_scale_exp(amax);
        uint32_t c[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          c[i] = e4m3x4(ldexpf(f[4 * i], -se), ldexpf(f[4 * i + 1], -se), ldexpf(f[4 * i + 2], -se),
                        ldexpf(f[4 * i + 3], -se));
        const uint4 codes = make_uint4(c[0], c[1], c[2], c[3]);
        // scale byte of the second block of this 64-wide step, from lane + 2
        const int se_hi = __shfl(se, (lane & ~3) + 2, 64);
        const uint16_t pair = (uint16_t)((se + 127) | ((se_hi + 127) << 8));
#pragma unroll
        for (int i = 0; i < kSlotGroup; ++i) {
          if (r[i] < 0) continue;  // remote slot
          buf_store16(rs[i], 16 * v, codes);
          if ((v & 3) == 0)  // pair plane v / 4, row r
            *reinterpret_cast<uint16_t*>(xs + (int64_t)(v >> 2) * xs_rows * 2 + (int64_t)r[i] * 2) = pair;
        }
      }
    }
  }
}

hipError_t launch_dispatch_gather_mxfp8(const void* x, const int32_t* row_of_pair, int T, int k, int d,
                                        uint8_t* xq, uint8_t* xs, int64_t xs_rows, int32_t* status, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int blocks = T < 16384 ? T : 16384;
  hipLaunchKernelGGL(dispatch_gather_mxfp8_kernel, dim3(blocks), dim3(256), 0, s, (const bf16_t*)x,
                     row_of_pair, T, k, d, xq, xs, xs_rows, status);
  return hipGetLastError();
}

// MXFP4 counterpart (E2M1 codes, two per byte, the lower element in the low
// nibble): 16 elements per lane, two lanes per MX block of 32, four per 64-wide
// K step; each lane writes its 8 code bytes, the first of four lanes the
// step's two scale bytes.
__global__ __launch_bounds__(256) void dispatch_gather_mxfp4_kernel(const bf16_t* __restrict__ x,
                                                                    const int32_t* __restrict__ rop, int ntok,
                                                                    int k, int d, uint8_t* __restrict__ xq,
                                                                    uint8_t* __restrict__ xs, int64_t xs_rows,
                                                                    int32_t* __restrict__ status) {
  const int nv = d / 16;
  const int lane = lane_id();
  for (int t = blockIdx.x; t < ntok; t += gridDim.x) {
    const int32_t* tr = rop + (int64_t)t * k;
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)t * d);
    for (int j0 = 0; j0 < k; j0 += kSlotGroup) {
      int32_t r[kSlotGroup];
      rsrc_t rs[kSlotGroup];
#pragma unroll
      for (int i = 0; i < kSlotGroup; ++i) {
        const int jc = j0 + i < k ? j0 + i : k - 1;
        const int32_t rv = checked_row(tr[jc], xs_rows, status);
        r[i] = (j0 + i < k) ? rv : -1;
        rs[i] = row_rsrc(xq, r[i], d / 2);
      }
      for (int v = threadIdx.x; v < nv; v += 256) {
        const uint4 w0 = src[2 * v], w1 = src[2 * v + 1];
        const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        float f[16];
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          f[2 * i] = __uint_as_float(w[i] << 16);
          f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
          amax = fmaxf(amax, fmaxf(fabsf(f[2 * i]), fabsf(f[2 * i + 1])));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
        const int se = mx4_scale_exp(amax);
        const uint2 codes = make_uint2(e2m1x8(f, se), e2m1x8(f + 8, se));
        const int se_hi = __shfl(se, (lane & ~3) + 2, 64);
        const uint16_t pair = (uint16_t)((se + 127) | ((se_hi + 127) << 8));
#pragma unroll
        for (int i = 0; i < kSlotGroup; ++i) {
          if (r[i] < 0) continue;  // remote slot
          buf_store8(rs[i], 8 * v, codes);
          if ((v & 3) == 0)  // pair plane v / 4, row r
            *reinterpret_cast<uint16_t*>(xs + (int64_t)(v >> 2) * xs_rows * 2 + (int64_t)r[i] * 2) = pair;
        }
      }
    }
  }
}

hipError_t launch_dispatch_gather_mxfp4(const void* x, const int32_t* row_of_pair, int T, int k, int d,
                                        uint8_t* xq, uint8_t* xs, int64_t xs_rows, int32_t* status, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int blocks = T < 16384 ? T : 16384;
  hipLaunchKernelGGL(dispatch_gather_mxfp4_kernel, dim3(blocks), dim3(256), 0, s, (const bf16_t*)x,
                     row_of_pair, T, k, d, xq, xs, xs_rows, status);
  return hipGetLastError();
}

// Quantise a [rows, K] bf16 matrix along its rows.  Vector i covers elements
// [8i, 8i + 8); K % 64 == 0 keeps each block of 32 (and each pair of blocks)
// inside one row.  Scales in pair planes: block b of row r at
// (b / 2) * 2 rows + 2 r + b % 2.
__global__ __launch_bounds__(256) void quantize_mxfp8_kernel(const bf16_t* __restrict__ src, int64_t nvec,
                                                             int64_t rows, int64_t K, uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ sc) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t iters = (nvec + stride - 1) / stride;
  for (int64_t it = 0; it < iters; ++it) {
    const int64_t v = it * stride + (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool act = v < nvec;
    uint4 val = act ? reinterpret_cast<const uint4*>(src)[v] : make_uint4(0, 0, 0, 0);
    uint2 codes;
    uint8_t sb;
    mx_quant8(val, codes, sb);
    if (act) {
      reinterpret_cast<uint2*>(q)[v] = codes;
      if ((v & 3) == 0) {
        const int64_t r = (8 * v) / K, b = ((8 * v) % K) / 32;
        sc[(b >> 1) * rows * 2 + r * 2 + (b & 1)] = sb;
      }
    }
  }
}

hipError_t launch_quantize_mxfp8(const void* src, int64_t rows, int64_t K, uint8_t* q, uint8_t* sc,
                                 hipStream_t s) {
  const int64_t nvec = rows * K / 8;
  if (nvec == 0) return hipSuccess;
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(quantize_mxfp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const bf16_t*)src, nvec,
                     rows, K, q, sc);
  return hipGetLastError();
}

// MXFP4 quantisation of a [rows, K] bf16 matrix along its rows: vector i
// covers elements [8i, 8i + 8) and becomes one dword of eight E2M1 codes
// (the lower element in the low nibble); scales as above.
__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(const bf16_t* __restrict__ src, int64_t nvec,
                                                             int64_t rows, int64_t K, uint32_t* __restrict__ q,
                                                             uint8_t* __restrict__ sc) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  const int64_t iters = (nvec + stride - 1) / stride;
  for (int64_t it = 0; it < iters; ++it) {
    const int64_t v = it * stride + (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool act = v < nvec;
    const uint4 val = act ? reinterpret_cast<const uint4*>(src)[v] : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {val.x, val.y, val.z, val.w};
    float f[8];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      amax = fmaxf(amax, fmaxf(fabsf(f[2 * i]), fabsf(f[2 * i + 1])));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const int se = mx4_scale_exp(amax);
    const uint32_t codes = e2m1x8(f, se);
    if (act) {
      q[v] = codes;
      if ((v & 3) == 0) {
        const int64_t r = (8 * v) / K, b = ((8 * v) % K) / 32;
        sc[(b >> 1) * rows * 2 + r * 2 + (b & 1)] = (uint8_t)(se + 127);
      }
    }
  }
}

hipError_t launch_quantize_mxfp4(const void* src, int64_t rows, int64_t K, uint8_t* q, uint8_t* sc,
                                 hipStream_t s) {
  const int64_t nvec = rows * K / 8;
  if (nvec == 0) return hipSuccess;
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(quantize_mxfp4_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const bf16_t*)src, nvec,
                     rows, K, (uint32_t*)q, sc);
  return hipGetLastError();
}

// Quantise the transpose of each [R, C] bf16 matrix of a batch along R:
// output row c of matrix m (global row m * C + c) holds the R values of
// source column c, as E4M3 codes at q + m * q_mat + c * q_ld + q_koff + r and
// E8M0 scales in pair planes of `rows` rows (K step (q_koff + r) / 64).
// One block per 64 x 64 tile, staged through LDS; four lanes per output row,
// 16 K values each (two lanes per MX block of 32).
__global__ __launch_bounds__(256) void quantize_mxfp8_t_kernel(const bf16_t* __restrict__ src, int R, int C,
                                                               uint8_t* __restrict__ q, int64_t q_mat,
                                                               int64_t q_ld, int q_koff,
                                                               uint8_t* __restrict__ sc, int64_t rows) {
  __shared__ float tile[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64, m = blockIdx.z;
  const bf16_t* s0 = src + (int64_t)m * R * C;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int v = it * 256 + threadIdx.x;  // 512 vectors of 8
    const int r = v >> 3, cv = (v & 7) * 8;
    const uint4 w = *reinterpret_cast<const uint4*>(s0 + (int64_t)(r0 + r) * C + c0 + cv);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[r][cv + 2 * i] = __uint_as_float(ww[i] << 16);
      tile[r][cv + 2 * i + 1] = __uint_as_float(ww[i] & 0xFFFF0000u);
    }
  }
  __syncthreads();
  const int c = threadIdx.x >> 2, qd = threadIdx.x & 3;
  float f[16];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    f[i] = tile[16 * qd + i][c];
    amax = fmaxf(amax, fabsf(f[i]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));  // lanes 2b, 2b + 1 share block b
  const int se = mx_scale_exp(amax);
  uint32_t cd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    cd[i] = e4m3x4(ldexpf(f[4 * i], -se), ldexpf(f[4 * i + 1], -se), ldexpf(f[4 * i + 2], -se),
                   ldexpf(f[4 * i + 3], -se));
  uint4 out;
  out.x = cd[0];
  out.y = cd[1];
  out.z = cd[2];
  out.w = cd[3];
  const int64_t orow = (int64_t)m * C + c0 + c;
  *reinterpret_cast<uint4*>(q + (int64_t)m * q_mat + (int64_t)(c0 + c) * q_ld + q_koff + r0 + 16 * qd) = out;
  if ((qd & 1) == 0) sc[(int64_t)((q_koff + r0) / 64) * rows * 2 + orow * 2 + (qd >> 1)] = (uint8_t)(se + 127);
}

hipError_t launch_quantize_mxfp8_t(const void* src, int nmat, int R, int C, uint8_t* q, int64_t q_mat,
                                   int64_t q_ld, int q_koff, uint8_t* sc, int64_t rows, hipStream_t s) {
  if (nmat == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_mxfp8_t_kernel, dim3(C / 64, R / 64, nmat), dim3(256), 0, s, (const bf16_t*)src, R,
                     C, q, q_mat, q_ld, q_koff, sc, rows);
  return hipGetLastError();
}

// ------------------------------------------------------------------ combine
// Raw 16-byte pieces of 8 elements: loaded first, widened to fp32 later, so
// that the loads of all rows a thread needs are in flight together.
template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
  struct Raw { uint4 v; };
  // elements [8v, 8v + 8) of a row
  __device__ static Raw load_raw(rsrc_t rs, int v) { return {buf_load16(rs, 16 * v)}; }
  __device__ static void widen(const Raw& r, float* f) {
    const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ static void load(const bf16_t* p, float* f) { widen({*reinterpret_cast<const uint4*>(p)}, f); }
  __device__ static void store(bf16_t* p, const float* f) {
    uint4 v;
    v.x = (uint32_t)f2bf(f[0]) | ((uint32_t)f2bf(f[1]) << 16);
    v.y = (uint32_t)f2bf(f[2]) | ((uint32_t)f2bf(f[3]) << 16);
    v.z = (uint32_t)f2bf(f[4]) | ((uint32_t)f2bf(f[5]) << 16);
    v.w = (uint32_t)f2bf(f[6]) | ((uint32_t)f2bf(f[7]) << 16);
    *reinterpret_cast<uint4*>(p) = v;
  }
  __device__ static void store(rsrc_t rs, int v, const float* f) {
    uint4 u;
    u.x = (uint32_t)f2bf(f[0]) | ((uint32_t)f2bf(f[1]) << 16);
    u.y = (uint32_t)f2bf(f[2]) | ((uint32_t)f2bf(f[3]) << 16);
    u.z = (uint32_t)f2bf(f[4]) | ((uint32_t)f2bf(f[5]) << 16);
    u.w = (uint32_t)f2bf(f[6]) | ((uint32_t)f2bf(f[7]) << 16);
    buf_store16(rs, 16 * v, u);
  }
};
template <> struct Vec8<float> {
  struct Raw { float4 a, b; };
  __device__ static Raw load_raw(rsrc_t rs, int v) {
    const uint4 a = buf_load16(rs, 32 * v), b = buf_load16(rs, 32 * v + 16);
    return {make_float4(__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z), __uint_as_float(a.w)),
            make_float4(__uint_as_float(b.x), __uint_as_float(b.y), __uint_as_float(b.z), __uint_as_float(b.w))};
  }
  __device__ static void widen(const Raw& r, float* f) {
    f[0] = r.a.x; f[1] = r.a.y; f[2] = r.a.z; f[3] = r.a.w; f[4] = r.b.x; f[5] = r.b.y; f[6] = r.b.z; f[7] = r.b.w;
  }
  __device__ static void load(const float* p, float* f) {
    widen({reinterpret_cast<const float4*>(p)[0], reinterpret_cast<const float4*>(p)[1]}, f);
  }
  __device__ static void store(float* p, const float* f) {
    reinterpret_cast<float4*>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
  }
  __device__ static void store(rsrc_t rs, int v, const float* f) {
    buf_store16(rs, 32 * v, make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                                       __float_as_uint(f[3])));
    buf_store16(rs, 32 * v + 16, make_uint4(__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]),
                                            __float_as_uint(f[7])));
  }
};

// In the combine, the kSlotGroup slots of a group are loaded before the first
// is used: a gather is bound by how many loads are in flight.

// out[t] = sum_{j ascending} w_j * rows[row(t,j)] in fp32, rounded once.
// w_j = gate[t,j], or 1 when gate is null (the reverse-dispatch reduction).
// Remote slots (row -1) are skipped.  The token's row indices and gates are
// the same for every lane, so they come through the scalar cache and no
// block barrier is needed.
template <typename T, bool GATED>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ rows, const float* __restrict__ gate,
                                                      const int32_t* __restrict__ rop, int ntok, int k, int d,
                                                      T* __restrict__ out, int64_t nrows,
                                                      int32_t* __restrict__ status) {
  const int nv = d / 8;
  for (int t = blockIdx.x; t < ntok; t += gridDim.x) {
    const int32_t* tr = rop + (int64_t)t * k;
    const float* tg = gate + (int64_t)t * k;
    // resources and weights of the first group, read once per token (the
    // loads are clamped to slot k - 1 so that they can all be issued at once)
    rsrc_t rs0[kSlotGroup];
    float w0[kSlotGroup];
#pragma unroll
    for (int i = 0; i < kSlotGroup; ++i) {
      const int jc = i < k ? i : k - 1;
      const int32_t rv = checked_row(tr[jc], nrows, status);
      const float gv = GATED ? tg[jc] : 1.0f;
      const int32_t r = (i < k) ? rv : -1;
      w0[i] = r < 0 ? 0.f : gv;
      rs0[i] = row_rsrc(rows, r, d * (int)sizeof(T));
    }
    for (int v = threadIdx.x; v < nv; v += 256) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < k; j0 += kSlotGroup) {
        typename Vec8<T>::Raw raw[kSlotGroup];
        float w[kSlotGroup];
#pragma unroll
        for (int i = 0; i < kSlotGroup; ++i) {
          rsrc_t rs = rs0[i];
          w[i] = w0[i];
          if (j0 > 0) {
            const int32_t r = (j0 + i < k) ? checked_row(tr[j0 + i], nrows, status) : -1;
            w[i] = r < 0 ? 0.f : (GATED ? tg[j0 + i] : 1.0f);
            rs = row_rsrc(rows, r, d * (int)sizeof(T));
          }
          raw[i] = Vec8<T>::load_raw(rs, v);
        }
        // a remote slot adds w * 0 = +-0 to an accumulator that is never -0:
        // the sum is the one over the local slots alone
#pragma unroll
        for (int i = 0; i < kSlotGroup; ++i) {
          float y[8];
          Vec8<T>::widen(raw[i], y);
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] = fmaf(w[i], y[q], acc[q]);
        }
      }
      Vec8<T>::store(out + (int64_t)t * d + 8 * v, acc);
    }
  }
}

// Calls that own a subset of the experts (an expert-parallel share) have
// mostly remote slots (about one local slot in eight per token at 4 of 256
// experts): there a block first lists the token's local rows in LDS and then
// reads only those (75 us against 104 us for the all-slots kernel on the
// share of experts 0-3 of 256, d 7168, 15,650 tokens).
template <typename T>
__global__ __launch_bounds__(256) void combine_compact_kernel(const T* __restrict__ rows, const float* __restrict__ gate,
                                                      const int32_t* __restrict__ rop, int ntok, int k, int d,
                                                      T* __restrict__ out, int64_t nrows,
                                                      int32_t* __restrict__ status) {
  __shared__ int32_t rr[kMaxK];
  __shared__ float ww[kMaxK];
  __shared__ int nloc;
  const int nv = d / 8;
  for (int t = blockIdx.x; t < ntok; t += gridDim.x) {
    if (threadIdx.x == 0) {
      int n = 0;
      for (int j = 0; j < k; ++j) {
        const int r = checked_row(rop[(int64_t)t * k + j], nrows, status);
        if (r >= 0) {
          rr[n] = r;
          ww[n] = gate ? gate[(int64_t)t * k + j] : 1.0f;
          ++n;
        }
      }
      nloc = n;
    }
    __syncthreads();
    const int n = nloc;
    for (int v = threadIdx.x; v < nv; v += 256) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < n; ++j) {
        float y[8];
        Vec8<T>::load(rows + (int64_t)rr[j] * d + 8 * v, y);
        const float w = ww[j];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = fmaf(w, y[q], acc[q]);
      }
      Vec8<T>::store(out + (int64_t)t * d + 8 * v, acc);
    }
    __syncthreads();
  }
}

hipError_t launch_combine(const void* rows, const float* gate, const int32_t* row_of_pair, int T, int k, int d,
                          int bf16, int all_local, void* out, int64_t nrows, int32_t* status, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int blocks = T < 16384 ? T : 16384;
  if (!all_local) {
    if (bf16)
      hipLaunchKernelGGL(combine_compact_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s, (const bf16_t*)rows, gate,
                         row_of_pair, T, k, d, (bf16_t*)out, nrows, status);
    else
      hipLaunchKernelGGL(combine_compact_kernel<float>, dim3(blocks), dim3(256), 0, s, (const float*)rows, gate,
                         row_of_pair, T, k, d, (float*)out, nrows, status);
    return hipGetLastError();
  }
#define MOK_COMBINE(TT, G)                                                                                 \
  hipLaunchKernelGGL((combine_kernel<TT, G>), dim3(blocks), dim3(256), 0, s, (const TT*)rows, gate, row_of_pair, T, \
                     k, d, (TT*)out, nrows, status)
  if (bf16) {
    if (gate) MOK_COMBINE(bf16_t, true); else MOK_COMBINE(bf16_t, false);
  } else {
    if (gate) MOK_COMBINE(float, true); else MOK_COMBINE(float, false);
  }
#undef MOK_COMBINE
  return hipGetLastError();
}

// ------------------------------------------------------------------ reverse-combine + router backward
// Per token: dgate_j = <dout_t, Y[row_j]> (fixed-order block reduction),
// dY[row_j] = gate_j * dout_t, then d(logits) by the router variant, with
// s = sum_j gate_j dgate_j (slot order) and G the dgate values at the chosen
// experts:
//   softmax:            dlogits = p * (G - s), p = exp(l - lse), every expert;
//   softmax, renorm:    gate_e * (G_e - s) at the chosen experts, 0 elsewhere;
//   sigmoid:            gate_e * (1 - sigmoid(l_e)) * G_e at the chosen experts;
//   sigmoid, renorm:    gate_e * (1 - sigmoid(l_e)) * (G_e - s) there.
// (With renorm, gate_j = a_j / S and d(a_i) = (G_i - s) / S; the softmax
// Jacobian then gives p_e (G_e - s) / S = gate_e (G_e - s) at the chosen
// experts and 0 elsewhere, since the chosen (G_i - s) average to zero under
// p; the sigmoid's derivative a (1 - a) gives the sigmoid lines.)
// MX: dY rows are also written as MXFP8 (E4M3 codes along d in dyq, E8M0
// scales in pair planes of dys_rows rows in dys), quantised from the fp32
// values gate * dout before their bf16 rounding.
template <typename T, int GATING, bool MX>
__global__ __launch_bounds__(256) void backward_gate_kernel(const T* __restrict__ dout, const T* __restrict__ Y,
                                                            const float* __restrict__ gate,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ rop,
                                                            const float* __restrict__ logits,
                                                            const float* __restrict__ lse, int ntok, int k, int E,
                                                            int d, float* __restrict__ dgate,
                                                            float* __restrict__ dlogits, T* __restrict__ dy,
                                                            int32_t* __restrict__ queue_zero, int nqueue,
                                                            uint8_t* __restrict__ dyq, uint8_t* __restrict__ dys,
                                                            int64_t dys_rows, int64_t nrows,
                                                            int32_t* __restrict__ status) {
  __shared__ float red[4][kSlotGroup];
  // the tile counters of the weight-gradient GEMMs that follow on the stream
  if (blockIdx.x == 0 && (int)threadIdx.x < nqueue) queue_zero[threadIdx.x] = 0;
  __shared__ float dg[kMaxK];
  __shared__ int32_t sel[kMaxK];
  const int nv = d / 8;
  const int lane = lane_id(), w = threadIdx.x >> 6;
  for (int t = blockIdx.x; t < ntok; t += gridDim.x) {
    const int32_t* tr = rop + (int64_t)t * k;
    const float* tg = gate + (int64_t)t * k;
    // Slots in groups: each thread's partial dot products of one group run
    // over its vectors in ascending order (v, then element), then one wave
    // sum and a fixed tree over the four waves.
    for (int j0 = 0; j0 < k; j0 += kSlotGroup) {
      int r[kSlotGroup];
      float g[kSlotGroup], part[kSlotGroup];
#pragma unroll
      for (int i = 0; i < kSlotGroup; ++i) {
        const int jc = j0 + i < k ? j0 + i : k - 1;  // clamped: all loads issued at once
        const int32_t rv = checked_row(tr[jc], nrows, status);
        const float gv = tg[jc];
        r[i] = (j0 + i < k) ? rv : -1;
        g[i] = (j0 + i < k) ? gv : 0.f;
        part[i] = 0.f;
      }
      rsrc_t yr[kSlotGroup], dyr[kSlotGroup];
#pragma unroll
      for (int i = 0; i < kSlotGroup; ++i) {
        yr[i] = row_rsrc(Y, r[i], d * (int)sizeof(T));
        dyr[i] = row_rsrc(dy, r[i], d * (int)sizeof(T));
      }
      for (int v = threadIdx.x; v < nv; v += 256) {
        typename Vec8<T>::Raw raw[kSlotGroup];
        float o[8];
        Vec8<T>::load(dout + (int64_t)t * d + 8 * v, o);
#pragma unroll
        for (int i = 0; i < kSlotGroup; ++i) raw[i] = Vec8<T>::load_raw(yr[i], v);
        // a remote slot reads zeros (its partial stays +0, reduced to 0 and
        // replaced by 0 below) and its store is dropped
#pragma unroll
        for (int i = 0; i < kSlotGroup; ++i) {
          float y[8], z[8];
          Vec8<T>::widen(raw[i], y);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            part[i] = fmaf(o[q], y[q], part[i]);
            z[q] = g[i] * o[q];
          }
          if (dy) Vec8<T>::store(dyr[i], v, z);  // no bf16 dY rows: MXFP8 codes only
          if constexpr (MX) {
            // lanes 4m .. 4m + 3 hold the 32 values of one block (d % 64 == 0
            // in MXFP8, so a group of eight lanes is active or inactive as a
            // whole)
            float amax = 0.f;
#pragma unroll
            for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(z[q]));
            amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
            amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
            const int se = mx_scale_exp(amax);
            // the second block of this 64-wide K step is four lanes up; the
            // two scale bytes are adjacent in the pair plane (d % 64 == 0)
            const int se_hi = __shfl(se, (lane & ~7) + 4, 64);
            const uint32_t c0 = e4m3x4(ldexpf(z[0], -se), ldexpf(z[1], -se), ldexpf(z[2], -se), ldexpf(z[3], -se));
            const uint32_t c1 = e4m3x4(ldexpf(z[4], -se), ldexpf(z[5], -se), ldexpf(z[6], -se), ldexpf(z[7], -se));
            if (r[i] >= 0) {
              uint2 codes;
              codes.x = c0;
              codes.y = c1;
              reinterpret_cast<uint2*>(dyq + (int64_t)r[i] * d)[v] = codes;
              if ((v & 7) == 0)
                *reinterpret_cast<uint16_t*>(dys + (int64_t)(v >> 3) * dys_rows * 2 + (int64_t)r[i] * 2) =
                    (uint16_t)((se + 127) | ((se_hi + 127) << 8));
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kSlotGroup; ++i) {
        const float ws = wave_sum(part[i]);
        if (lane == 0) red[w][i] = ws;
      }
      __syncthreads();
      if ((int)threadIdx.x < kSlotGroup && j0 + (int)threadIdx.x < k) {
        const int i = threadIdx.x, j = j0 + i;
        const int rj = checked_row(tr[j], nrows, status);
        dg[j] = (rj >= 0) ? ((red[0][i] + red[1][i]) + (red[2][i] + red[3][i])) : 0.f;
        const int32_t ej = idx[(int64_t)t * k + j];
        if (ej < 0 || ej >= E) report(status, kCheckIndex);  // only compared below: no access through it
        sel[j] = ej;
      }
      __syncthreads();
    }
    constexpr bool SIGM = GATING & kGateSigmoid, RENORM = GATING & kGateRenorm;
    float s = 0.f;
    if (!SIGM || RENORM)
      for (int j = 0; j < k; ++j) s = fmaf(gate[(int64_t)t * k + j], dg[j], s);
    for (int j = threadIdx.x; j < k; j += 256) dgate[(int64_t)t * k + j] = dg[j];
    const float l0 = lse[t];
    for (int e = threadIdx.x; e < E; e += 256) {
      const float l = logits[(int64_t)t * E + e];
      float G = 0.f, ge = 0.f;
      bool chosen = false;
      for (int j = 0; j < k; ++j)
        if (sel[j] == e) {
          G = dg[j];
          ge = gate[(int64_t)t * k + j];
          chosen = true;
        }
      float out;
      if constexpr (!SIGM && !RENORM) {
        out = expf(l - l0) * (G - s);
      } else if (!chosen) {
        out = 0.f;
      } else {
        const float c = SIGM ? 1.0f - 1.0f / (1.0f + expf(-l)) : 1.0f;
        out = ge * c * (G - s);
      }
      dlogits[(int64_t)t * E + e] = out;
    }
    __syncthreads();
  }
}

hipError_t launch_backward_gate(const void* dout, const void* Y, const float* gate, const int32_t* idx,
                                const int32_t* row_of_pair, const float* logits, const float* lse, int T, int k,
                                int E, int d, int gating, int bf16, float* dgate, float* dlogits, void* dy,
                                int32_t* queue_zero, int nqueue, uint8_t* dyq, uint8_t* dys, int64_t dys_rows,
                                int64_t nrows, int32_t* status, hipStream_t s) {
  int blocks = T < 16384 ? (T > 0 ? T : 1) : 16384;  // at least one block: it zeroes the counters
  if (!dy && !dyq) return hipErrorInvalidValue;  // dY goes somewhere
#define MOK_BWD_GATE(TT, GV, MXV)                                                                              \
  hipLaunchKernelGGL((backward_gate_kernel<TT, GV, MXV>), dim3(blocks), dim3(256), 0, s, (const TT*)dout,      \
                     (const TT*)Y, gate, idx, row_of_pair, logits, lse, T, k, E, d, dgate, dlogits, (TT*)dy,    \
                     queue_zero, nqueue, dyq, dys, dys_rows, nrows, status)
#define MOK_BWD_GATE_T(TT, MXV)                                         \
  switch (gating & (kGateSigmoid | kGateRenorm)) {                      \
    case 0: MOK_BWD_GATE(TT, 0, MXV); break;                            \
    case kGateSigmoid: MOK_BWD_GATE(TT, kGateSigmoid, MXV); break;      \
    case kGateRenorm: MOK_BWD_GATE(TT, kGateRenorm, MXV); break;        \
    default: MOK_BWD_GATE(TT, kGateSigmoid | kGateRenorm, MXV); break; \
  }
  if (dyq) {
    if (!bf16) return hipErrorInvalidValue;
    MOK_BWD_GATE_T(bf16_t, true)
  } else if (bf16) {
    MOK_BWD_GATE_T(bf16_t, false)
  } else {
    MOK_BWD_GATE_T(float, false)
  }
#undef MOK_BWD_GATE_T
#undef MOK_BWD_GATE
  return hipGetLastError();
}

}  // namespace mok
