// Expert-grouped fp32 GEMMs (vector ALU, LDS-tiled) for the fp32 precision of
// the layer: the same six products and epilogues as the BF16 MFMA kernels
// (kucoin.com, "Cursor's MoK réalise une amélioration des performances de
// 2,37x sur NVIDIA GB300 NVL72", sections 01 and 02: grouped expert GEMMs,
// SwiGLU).  A workgroup of 256 threads computes a 64 x 64 tile, 4 x 4 outputs
// per thread, K in steps of 16 through LDS; one workgroup per output element
// and a fixed K order keep results run-to-run identical.
#include "mok_device.h"
#include "mok_internal.h"
#include "gemm_common.h"

namespace mok {

template <int KIND>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(GroupedGemmArgs args) {
  using Tr = Traits<KIND>;
  constexpr int BM = 64, BN = 64, BK = 16, NB = Tr::NB;
  __shared__ float sA[BK][BM + 4];
  __shared__ float sB[NB][BK][BN + 4];
  __shared__ int32_t s_tp[1025];

  const GemmGeom G = geom_of<KIND>(args.d, args.F);
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const float* __restrict__ Abase = (const float*)args.A;
  const float* __restrict__ B0 = (const float*)args.B0;
  const float* __restrict__ B1 = (const float*)args.B1;
  const int E_loc = args.E_loc;
  const int ntn = (G.N + BN - 1) / BN;
  int total, ntm_k = 0;
  if constexpr (!Tr::GROUP_K) {
    const int32_t* tp = args.tile_prefix;  // BM = 64 table
    for (int i = tid; i <= E_loc; i += 256) s_tp[i] = tp[i];
    __syncthreads();
    total = s_tp[E_loc] * ntn;
  } else {
    ntm_k = (G.M + BM - 1) / BM;
    total = E_loc * ntm_k * ntn;
  }
  const int z = KIND == KIND_DW13 ? blockIdx.y : 0;

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    int e_loc, row0, row_end, m0 = 0, n0;
    if constexpr (!Tr::GROUP_K) {
      const int total_m = s_tp[E_loc];
      const int mt = tile % total_m;
      n0 = (tile / total_m) * BN;
      int lo = 0, hi = E_loc - 1;
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (s_tp[mid] <= mt) lo = mid; else hi = mid - 1;
      }
      e_loc = lo;
      row0 = args.offsets[args.eb + e_loc] + (mt - s_tp[e_loc]) * BM;
      row_end = args.offsets[args.eb + e_loc + 1];
    } else {
      e_loc = tile / (ntm_k * ntn);
      const int rem = tile % (ntm_k * ntn);
      m0 = (rem % ntm_k) * BM;
      n0 = (rem / ntm_k) * BN;
      row0 = args.offsets[args.eb + e_loc];
      row_end = args.offsets[args.eb + e_loc + 1];
    }
    const int kbeg = Tr::GROUP_K ? row0 : 0;
    const int kend = Tr::GROUP_K ? row_end : G.K;

    float acc[NB][4][4];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[b][i][j] = 0.f;

    for (int k0 = kbeg; k0 < kend; k0 += BK) {
      // A tile: 64 x 16 = 1024 values, 4 per thread
      {
        float v[4];
        int dst_k, dst_m;
        if constexpr (!Tr::A_MN) {
          const int i = tid / 4, kc = (tid % 4) * 4;
          int r = row0 + i;
          r = r < row_end ? r : row_end - 1;
          const float4 f = *reinterpret_cast<const float4*>(Abase + (int64_t)r * G.lda + k0 + kc);
          v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
#pragma unroll
          for (int q = 0; q < 4; ++q) sA[kc + q][i] = v[q];
          (void)dst_k; (void)dst_m;
        } else {
          const int kk = tid / 16, mc = (tid % 16) * 4;
          const int kr = k0 + kk, m = m0 + mc;
          const float* p = Abase + (KIND == KIND_DW13 ? (int64_t)z * args.F : 0);
          float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
          if (kr < kend && m < G.M) f = *reinterpret_cast<const float4*>(p + (int64_t)kr * G.lda + m);
          sA[kk][mc] = f.x; sA[kk][mc + 1] = f.y; sA[kk][mc + 2] = f.z; sA[kk][mc + 3] = f.w;
        }
      }
      // B tile(s)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if constexpr (!Tr::B_MN) {
          const int i = tid / 4, kc = (tid % 4) * 4;
          int n = n0 + i;
          n = n < G.N ? n : G.N - 1;
          const float* base = (b ? B1 : B0) + (int64_t)e_loc * G.b_estride;
          const float4 f = *reinterpret_cast<const float4*>(base + (int64_t)n * G.ldb + k0 + kc);
          sB[b][kc][i] = f.x; sB[b][kc + 1][i] = f.y; sB[b][kc + 2][i] = f.z; sB[b][kc + 3][i] = f.w;
        } else if constexpr (!Tr::GROUP_K) {
          const int kk = tid / 16, nc = (tid % 16) * 4;
          const int kr = k0 + kk, n = n0 + nc;
          const float* base = (kr < G.ksplit ? B0 : B1) + (int64_t)e_loc * G.b_estride;
          const int krl = kr < G.ksplit ? kr : kr - G.ksplit;
          float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
          if (n < G.N) f = *reinterpret_cast<const float4*>(base + (int64_t)krl * G.ldb + n);
          sB[b][kk][nc] = f.x; sB[b][kk][nc + 1] = f.y; sB[b][kk][nc + 2] = f.z; sB[b][kk][nc + 3] = f.w;
        } else {
          const int kk = tid / 16, nc = (tid % 16) * 4;
          const int kr = k0 + kk, n = n0 + nc;
          float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
          if (kr < kend && n < G.N) f = *reinterpret_cast<const float4*>(B0 + (int64_t)kr * G.ldb + n);
          sB[b][kk][nc] = f.x; sB[b][kk][nc + 1] = f.y; sB[b][kk][nc + 2] = f.z; sB[b][kk][nc + 3] = f.w;
        }
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float a[4], bv[NB][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int j = 0; j < 4; ++j) bv[b][j] = sB[b][kk][tx * 4 + j];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[b][i][j] = fmaf(a[i], bv[b][j], acc[b][i][j]);
      }
      __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rit = ty * 4 + i, col = n0 + tx * 4 + j;
        if (col >= G.N) continue;
        const float v = acc[0][i][j];
        if constexpr (!Tr::GROUP_K) {
          const int row = row0 + rit;
          if (row >= row_end) continue;
          if constexpr (KIND == KIND_UP) {
            const float u = acc[NB - 1][i][j];
            ((float*)args.out0)[(int64_t)row * G.N + col] = v * sigmoidf_(v) * u;
            if (args.save) {
              ((float*)args.save_a)[(int64_t)row * G.N + col] = v;
              ((float*)args.save_b)[(int64_t)row * G.N + col] = u;
            }
          } else if constexpr (KIND == KIND_DH) {
            const float a = ((const float*)args.save_a)[(int64_t)row * G.N + col];
            const float b = ((const float*)args.save_b)[(int64_t)row * G.N + col];
            const float sg = sigmoidf_(a);
            float* dab = (float*)args.out0 + (int64_t)row * 2 * args.F;
            dab[col] = v * b * sg * (1.0f + a * (1.0f - sg));
            dab[args.F + col] = v * a * sg;
          } else {
            ((float*)args.out0)[(int64_t)row * G.N + col] = v;
          }
        } else {
          const int m = m0 + rit;
          if (m >= G.M) continue;
          float* outp = (float*)(KIND == KIND_DW13 && z ? args.out1 : args.out0);
          outp[(int64_t)e_loc * G.M * G.N + (int64_t)m * G.N + col] = v;
        }
      }
    }
  }
}

template <int KIND>
static hipError_t run_f32(const GroupedGemmArgs& g, hipStream_t s) {
  const GemmGeom G = geom_of<KIND>(g.d, g.F);
  const int ntn = (G.N + 63) / 64;
  int blocks;
  dim3 grid;
  if constexpr (Traits<KIND>::GROUP_K) {
    blocks = g.E_loc * ((G.M + 63) / 64) * ntn;
    grid = dim3(blocks, KIND == KIND_DW13 ? 2 : 1);
  } else {
    const int64_t worst = ((g.P_max + 63) / 64 + g.E_loc) * (int64_t)ntn;
    blocks = (int)(worst < 2048 ? worst : 2048);
    grid = dim3(blocks);
  }
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_gemm_f32_kernel<KIND>, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t gemm_f32(int kind, const GroupedGemmArgs& g, hipStream_t s) {
  switch (kind) {
    case KIND_UP:   return run_f32<KIND_UP>(g, s);
    case KIND_DOWN: return run_f32<KIND_DOWN>(g, s);
    case KIND_DH:   return run_f32<KIND_DH>(g, s);
    case KIND_DX:   return run_f32<KIND_DX>(g, s);
    case KIND_DW2:  return run_f32<KIND_DW2>(g, s);
    case KIND_DW13: return run_f32<KIND_DW13>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mok
