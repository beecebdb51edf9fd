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

// ------------------------------------------------------------------ dispatch
// One block per token: read x[t] once (16-byte vectors), write it to the
// rows of its local pairs.
template <typename T>
__global__ __launch_bounds__(256) void dispatch_gather_kernel(const T* __restrict__ x,
                                                              const int32_t* __restrict__ rop, int ntok,
                                                              int k, int d, T* __restrict__ xp) {
  __shared__ int32_t rows[kMaxK];
  __shared__ int nloc;
  const int nv = d * (int)sizeof(T) / 16;
  for (int t = blockIdx.x; t < ntok; t += gridDim.x) {
    if (threadIdx.x == 0) {
      int n = 0;
      for (int j = 0; j < k; ++j) {
        int r = rop[(int64_t)t * k + j];
        if (r >= 0) rows[n++] = r;
      }
      nloc = n;
    }
    __syncthreads();
    const int n = nloc;
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)t * d);
    for (int v = threadIdx.x; v < nv; v += 256) {
      uint4 val = src[v];
      for (int j = 0; j < n; ++j) reinterpret_cast<uint4*>(xp + (int64_t)rows[j] * d)[v] = val;
    }
    __syncthreads();
  }
}

hipError_t launch_dispatch_gather(const void* x, const int32_t* row_of_pair, int T, int k, int d, int bf16,
                                  void* xp, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int blocks = T < 16384 ? T : 16384;
  if (bf16)
    hipLaunchKernelGGL(dispatch_gather_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s,
                       (const bf16_t*)x, row_of_pair, T, k, d, (bf16_t*)xp);
  else
    hipLaunchKernelGGL(dispatch_gather_kernel<float>, dim3(blocks), dim3(256), 0, s, (const float*)x,
                       row_of_pair, T, k, d, (float*)xp);
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
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = e4m3_rne(ldexpf(f[i], -se));
  codes.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
  codes.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
  scale_byte = (uint8_t)(se + 127);
}

__global__ __launch_bounds__(256) void dispatch_gather_mxfp8_kernel(const bf16_t* __restrict__ x,
                                                                    const int32_t* __restrict__ rop, int ntok,
                                                                    int k, int d, uint8_t* __restrict__ xq,
                                                                    uint8_t* __restrict__ xs, int64_t xs_rows) {
  __shared__ int32_t rows[kMaxK];
  __shared__ int nloc;
  const int nv = d / 8;            // multiple of 4: blocks of 32 never straddle lanes groups
  const int iters = (nv + 255) / 256;
  for (int t = blockIdx.x; t < ntok; t += gridDim.x) {
    if (threadIdx.x == 0) {
      int n = 0;
      for (int j = 0; j < k; ++j) {
        int r = rop[(int64_t)t * k + j];
        if (r >= 0) rows[n++] = r;
      }
      nloc = n;
    }
    __syncthreads();
    const int n = nloc;
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)t * d);
    for (int it = 0; it < iters; ++it) {
      const int v = it * 256 + threadIdx.x;
      const bool act = v < nv;
      uint4 val = act ? src[v] : make_uint4(0, 0, 0, 0);
      uint2 codes;
      uint8_t sb;
      mx_quant8(val, codes, sb);
      if (act) {
        for (int j = 0; j < n; ++j) {
          reinterpret_cast<uint2*>(xq + (int64_t)rows[j] * d)[v] = codes;
          if ((v & 3) == 0) {  // pair-plane scale layout, xs_rows rows per plane
            const int b = v >> 2;
            xs[(int64_t)(b >> 1) * xs_rows * 2 + (int64_t)rows[j] * 2 + (b & 1)] = sb;
          }
        }
      }
    }
    __syncthreads();
  }
}

hipError_t launch_dispatch_gather_mxfp8(const void* x, const int32_t* row_of_pair, int T, int k, int d,
                                        uint8_t* xq, uint8_t* xs, int64_t xs_rows, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int blocks = T < 16384 ? T : 16384;
  hipLaunchKernelGGL(dispatch_gather_mxfp8_kernel, dim3(blocks), dim3(256), 0, s, (const bf16_t*)x,
                     row_of_pair, T, k, d, xq, xs, xs_rows);
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

// ------------------------------------------------------------------ combine
template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
  __device__ static void load(const bf16_t* p, float* f) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ static void store(bf16_t* p, const float* f) {
    uint4 v;
    v.x = (uint32_t)f2bf(f[0]) | ((uint32_t)f2bf(f[1]) << 16);
    v.y = (uint32_t)f2bf(f[2]) | ((uint32_t)f2bf(f[3]) << 16);
    v.z = (uint32_t)f2bf(f[4]) | ((uint32_t)f2bf(f[5]) << 16);
    v.w = (uint32_t)f2bf(f[6]) | ((uint32_t)f2bf(f[7]) << 16);
    *reinterpret_cast<uint4*>(p) = v;
  }
};
template <> struct Vec8<float> {
  __device__ static void load(const float* p, float* f) {
    float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  __device__ static void store(float* p, const float* f) {
    reinterpret_cast<float4*>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
  }
};

// out[t] = sum_{j ascending} w_j * rows[row(t,j)] in fp32, rounded once.
// w_j = gate[t,j], or 1 when gate is null (the reverse-dispatch reduction).
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ rows, const float* __restrict__ gate,
                                                      const int32_t* __restrict__ rop, int ntok, int k, int d,
                                                      T* __restrict__ out) {
  __shared__ int32_t rr[kMaxK];
  __shared__ float ww[kMaxK];
  __shared__ int nloc;
  const int nv = d / 8;
  for (int t = blockIdx.x; t < ntok; t += gridDim.x) {
    if (threadIdx.x == 0) {
      int n = 0;
      for (int j = 0; j < k; ++j) {
        int r = rop[(int64_t)t * k + j];
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
                          int bf16, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int blocks = T < 16384 ? T : 16384;
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s, (const bf16_t*)rows, gate,
                       row_of_pair, T, k, d, (bf16_t*)out);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(blocks), dim3(256), 0, s, (const float*)rows, gate,
                       row_of_pair, T, k, d, (float*)out);
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
template <typename T, int GATING>
__global__ __launch_bounds__(256) void backward_gate_kernel(const T* __restrict__ dout, const T* __restrict__ Y,
                                                            const float* __restrict__ gate,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ rop,
                                                            const float* __restrict__ logits,
                                                            const float* __restrict__ lse, int ntok, int k, int E,
                                                            int d, float* __restrict__ dgate,
                                                            float* __restrict__ dlogits, T* __restrict__ dy,
                                                            int32_t* __restrict__ queue_zero, int nqueue) {
  __shared__ float red[4];
  // the tile counters of the weight-gradient GEMMs that follow on the stream
  if (blockIdx.x == 0 && (int)threadIdx.x < nqueue) queue_zero[threadIdx.x] = 0;
  __shared__ float dg[kMaxK];
  __shared__ int32_t sel[kMaxK];
  const int nv = d / 8;
  const int lane = lane_id(), w = threadIdx.x >> 6;
  for (int t = blockIdx.x; t < ntok; t += gridDim.x) {
    for (int j = 0; j < k; ++j) {
      const int r = rop[(int64_t)t * k + j];
      const float g = gate[(int64_t)t * k + j];
      float part = 0.f;
      if (r >= 0) {
        for (int v = threadIdx.x; v < nv; v += 256) {
          float o[8], y[8], z[8];
          Vec8<T>::load(dout + (int64_t)t * d + 8 * v, o);
          Vec8<T>::load(Y + (int64_t)r * d + 8 * v, y);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            part = fmaf(o[q], y[q], part);
            z[q] = g * o[q];
          }
          Vec8<T>::store(dy + (int64_t)r * d + 8 * v, z);
        }
      }
      part = wave_sum(part);
      if (lane == 0) red[w] = part;
      __syncthreads();
      if (threadIdx.x == 0) {
        dg[j] = (r >= 0) ? ((red[0] + red[1]) + (red[2] + red[3])) : 0.f;
        sel[j] = idx[(int64_t)t * k + j];
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
                                int32_t* queue_zero, int nqueue, hipStream_t s) {
  int blocks = T < 16384 ? (T > 0 ? T : 1) : 16384;  // at least one block: it zeroes the counters
#define MOK_BWD_GATE(TT, GV)                                                                                     \
  hipLaunchKernelGGL((backward_gate_kernel<TT, GV>), dim3(blocks), dim3(256), 0, s, (const TT*)dout, (const TT*)Y, \
                     gate, idx, row_of_pair, logits, lse, T, k, E, d, dgate, dlogits, (TT*)dy, queue_zero, nqueue)
#define MOK_BWD_GATE_T(TT)                                         \
  switch (gating & (kGateSigmoid | kGateRenorm)) {                 \
    case 0: MOK_BWD_GATE(TT, 0); break;                            \
    case kGateSigmoid: MOK_BWD_GATE(TT, kGateSigmoid); break;      \
    case kGateRenorm: MOK_BWD_GATE(TT, kGateRenorm); break;        \
    default: MOK_BWD_GATE(TT, kGateSigmoid | kGateRenorm); break; \
  }
  if (bf16) {
    MOK_BWD_GATE_T(bf16_t)
  } else {
    MOK_BWD_GATE_T(float)
  }
#undef MOK_BWD_GATE_T
#undef MOK_BWD_GATE
  return hipGetLastError();
}

}  // namespace mok
