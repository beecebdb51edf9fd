// Expert-grouped BF16 GEMMs on MFMA (gfx950 v_mfma_f32_32x32x16_bf16), forward
// and backward, with fused epilogues.
//
// The expert FFNs run as a grouped GEMM over expert-contiguous rows, which is
// what keeps the matrix cores fed (kucoin.com, "Cursor's MoK réalise une
// amélioration des performances de 2,37x sur NVIDIA GB300 NVL72", section 01);
// the expert activation is SwiGLU (same page, section 02).  Forward and
// backward products of one expert e over its rows X_e (R_e x d):
//   UP    H_e   = silu(X_e W1_e^T) * (X_e W3_e^T)    [R_e, F]  (A, B saved)
//   DOWN  Y_e   = H_e W2_e^T                         [R_e, d]
//   DH    dH_e  = dY_e W2_e  -> dA, dB via SwiGLU'   [R_e, F] each
//   DX    dX_e  = dA_e W1_e + dB_e W3_e              [R_e, d]
//   DW2   dW2_e = dY_e^T H_e                         [d, F] fp32
//   DW13  dW1_e = dA_e^T X_e, dW3_e = dB_e^T X_e     [F, d] fp32
//
// Tiling: a workgroup computes a BM x BN output tile with WM x WN waves, each
// wave a (BM/WM) x (BN/WN) block of 32x32 MFMA tiles, over K in steps of BK
// staged through double-buffered LDS (K-contiguous [row][k] layout, padded).
// Row-grouped kinds walk a persistent loop over the tiles of all local experts;
// the per-expert tile prefix comes from the counting sort on the device, so
// the host never needs the data-dependent row count.  Every output element is
// produced by one workgroup with a fixed K order: results are run-to-run
// identical (no split-K, no atomics).
#include "mok_device.h"
#include "mok_internal.h"
#include "gemm_common.h"

namespace mok {

// Row-grouped epilogues: one output element (row, col) from the fp32
// accumulator v (and u, the W3 accumulator, for UP).
template <int KIND>
__device__ __forceinline__ void epilogue_rows(const GroupedGemmArgs& args, const GemmGeom& G, int row, int col,
                                              float v, float u) {
  const int64_t o = (int64_t)row * G.N + col;
  if constexpr (KIND == KIND_UP) {
    ((bf16_t*)args.out0)[o] = f2bf(v * sigmoidf_(v) * u);
    if (args.save) {
      ((bf16_t*)args.save_a)[o] = f2bf(v);
      ((bf16_t*)args.save_b)[o] = f2bf(u);
    }
  } else if constexpr (KIND == KIND_DH) {
    const float a = bf2f(((const bf16_t*)args.save_a)[o]);
    const float b = bf2f(((const bf16_t*)args.save_b)[o]);
    const float sg = sigmoidf_(a);
    bf16_t* dab = (bf16_t*)args.out0 + (int64_t)row * 2 * args.F;
    dab[col] = f2bf(v * b * sg * (1.0f + a * (1.0f - sg)));
    dab[args.F + col] = f2bf(v * a * sg);
  } else {
    ((bf16_t*)args.out0)[o] = f2bf(v);
  }
}

template <int BM, int BN, int BK, int WM, int WN, int KIND>
__global__ __launch_bounds__(WM * WN * 64) void grouped_gemm_bf16_kernel(GroupedGemmArgs args) {
  using Tr = Traits<KIND>;
  constexpr int NT = WM * WN * 64;
  constexpr int NB = Tr::NB;
  constexpr int PAD = 8;
  constexpr int LDS_K = BK + PAD;           // row stride in elements
  constexpr int TM = BM / WM, TN = BN / WN; // wave tile
  constexpr int FM = TM / 32, FN = TN / 32; // 32x32 MFMA tiles per wave
  constexpr int BROWS = NB * BN;
  static_assert(TM % 32 == 0 && TN % 32 == 0 && BK % 16 == 0, "bad tile");
  constexpr int CHA = BM * BK / 8 / NT;
  constexpr int CHB = BROWS * BK / 8 / NT;
  static_assert(BM * BK / 8 % NT == 0 && BROWS * BK / 8 % NT == 0, "tile must split evenly");

  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * LDS_K];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BROWS * LDS_K];
  __shared__ int32_t s_tp[1025];

  const GemmGeom G = geom_of<KIND>(args.d, args.F);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;
  const bf16_t* __restrict__ Abase = (const bf16_t*)args.A;
  const bf16_t* __restrict__ B0 = (const bf16_t*)args.B0;
  const bf16_t* __restrict__ B1 = (const bf16_t*)args.B1;
  const int E_loc = args.E_loc;

  // ---------------------------------------------------------------- tiles
  int total;
  int ntn = (G.N + BN - 1) / BN;
  int ntm_k = 0;  // GROUP_K: m tiles per expert
  if constexpr (!Tr::GROUP_K) {
    const int bidx = (BM == 64) ? 0 : (BM == 128 ? 1 : 2);
    const int32_t* tp = args.tile_prefix + bidx * (E_loc + 1);
    for (int i = tid; i <= E_loc; i += NT) s_tp[i] = tp[i];
    __syncthreads();
    total = s_tp[E_loc] * ntn;
  } else {
    ntm_k = (G.M + BM - 1) / BM;
    total = E_loc * ntm_k * ntn;
  }

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    int e_loc, row0, row_end, m0 = 0, n0;
    if constexpr (!Tr::GROUP_K) {
      const int total_m = s_tp[E_loc];
      const int mt = tile % total_m;
      n0 = (tile / total_m) * BN;
      int lo = 0, hi = E_loc - 1;  // largest i with s_tp[i] <= mt
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (s_tp[mid] <= mt) lo = mid; else hi = mid - 1;
      }
      e_loc = lo;
      const int e = args.eb + e_loc;
      row0 = args.offsets[e] + (mt - s_tp[e_loc]) * BM;
      row_end = args.offsets[e + 1];
    } else {
      e_loc = tile / (ntm_k * ntn);
      const int rem = tile % (ntm_k * ntn);
      m0 = (rem % ntm_k) * BM;
      n0 = (rem / ntm_k) * BN;
      const int e = args.eb + e_loc;
      row0 = args.offsets[e];
      row_end = args.offsets[e + 1];
    }
    const int z = KIND == KIND_DW13 ? blockIdx.y : 0;

    // K extent
    const int kbeg = Tr::GROUP_K ? row0 : 0;
    const int kend = Tr::GROUP_K ? row_end : G.K;
    const int nk = (kend - kbeg + BK - 1) / BK;

    u32x4_t ra[CHA], rb[CHB];

    auto load_a = [&](int k0) {
#pragma unroll
      for (int q = 0; q < CHA; ++q) {
        const int c = tid + q * NT;
        if constexpr (!Tr::A_MN) {
          const int i = c / (BK / 8), kc = c % (BK / 8);
          int r = row0 + i;
          r = r < row_end ? r : row_end - 1;
          ra[q] = *reinterpret_cast<const u32x4_t*>(Abase + (int64_t)r * G.lda + k0 + kc * 8);
        } else {
          const int kk = c / (BM / 8), mc = c % (BM / 8);
          const int kr = k0 + kk, m = m0 + mc * 8;
          const bf16_t* p = Abase + (KIND == KIND_DW13 ? (int64_t)z * args.F : 0);
          ra[q] = (kr < kend && m < G.M) ? *reinterpret_cast<const u32x4_t*>(p + (int64_t)kr * G.lda + m)
                                         : u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    };
    auto load_b = [&](int k0) {
#pragma unroll
      for (int q = 0; q < CHB; ++q) {
        const int c = tid + q * NT;
        if constexpr (!Tr::B_MN) {
          const int i = c / (BK / 8), kc = c % (BK / 8);
          const int which = (NB == 2 && i >= BN) ? 1 : 0;
          int n = n0 + i - which * BN;
          n = n < G.N ? n : G.N - 1;
          const bf16_t* base = (which ? B1 : B0) + (int64_t)e_loc * G.b_estride;
          rb[q] = *reinterpret_cast<const u32x4_t*>(base + (int64_t)n * G.ldb + k0 + kc * 8);
        } else if constexpr (!Tr::GROUP_K) {
          const int kk = c / (BN / 8), nc = c % (BN / 8);
          const int kr = k0 + kk, n = n0 + nc * 8;
          const bf16_t* base = (kr < G.ksplit ? B0 : B1) + (int64_t)e_loc * G.b_estride;
          const int krl = kr < G.ksplit ? kr : kr - G.ksplit;
          rb[q] = n < G.N ? *reinterpret_cast<const u32x4_t*>(base + (int64_t)krl * G.ldb + n)
                          : u32x4_t{0u, 0u, 0u, 0u};
        } else {
          const int kk = c / (BN / 8), nc = c % (BN / 8);
          const int kr = k0 + kk, n = n0 + nc * 8;
          rb[q] = (kr < kend && n < G.N) ? *reinterpret_cast<const u32x4_t*>(B0 + (int64_t)kr * G.ldb + n)
                                         : u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    };
    auto store_a = [&](int buf) {
#pragma unroll
      for (int q = 0; q < CHA; ++q) {
        const int c = tid + q * NT;
        if constexpr (!Tr::A_MN) {
          const int i = c / (BK / 8), kc = c % (BK / 8);
          *reinterpret_cast<u32x4_t*>(&sA[buf][i * LDS_K + kc * 8]) = ra[q];
        } else {
          const int kk = c / (BM / 8), mc = c % (BM / 8);
          const u32x4_t w = ra[q];
#pragma unroll
          for (int h = 0; h < 8; ++h)
            sA[buf][(mc * 8 + h) * LDS_K + kk] = (bf16_t)((h & 1) ? (w[h >> 1] >> 16) : (w[h >> 1] & 0xFFFF));
        }
      }
    };
    auto store_b = [&](int buf) {
#pragma unroll
      for (int q = 0; q < CHB; ++q) {
        const int c = tid + q * NT;
        if constexpr (!Tr::B_MN) {
          const int i = c / (BK / 8), kc = c % (BK / 8);
          *reinterpret_cast<u32x4_t*>(&sB[buf][i * LDS_K + kc * 8]) = rb[q];
        } else {
          const int kk = c / (BN / 8), nc = c % (BN / 8);
          const u32x4_t w = rb[q];
#pragma unroll
          for (int h = 0; h < 8; ++h)
            sB[buf][(nc * 8 + h) * LDS_K + kk] = (bf16_t)((h & 1) ? (w[h >> 1] >> 16) : (w[h >> 1] & 0xFFFF));
        }
      }
    };

    f32x16_t acc[NB][FM][FN];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[b][i][j][r] = 0.f;

    if (nk > 0) {
      load_a(kbeg);
      load_b(kbeg);
      store_a(0);
      store_b(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) {
        load_a(kbeg + (kt + 1) * BK);
        load_b(kbeg + (kt + 1) * BK);
      }
      const bf16_t* a_s = sA[buf];
      const bf16_t* b_s = sB[buf];
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int koff = kk * 16 + (lane >> 5) * 8;
        bf16x8_t af[FM], bfr[NB][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[i] = *reinterpret_cast<const bf16x8_t*>(&a_s[(wm * TM + i * 32 + (lane & 31)) * LDS_K + koff]);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            bfr[b][j] = *reinterpret_cast<const bf16x8_t*>(
                &b_s[(b * BN + wn * TN + j * 32 + (lane & 31)) * LDS_K + koff]);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
              acc[b][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[b][j], acc[b][i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) {
        store_a(buf ^ 1);
        store_b(buf ^ 1);
      }
      __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * TN + j * 32 + (lane & 31);
        const bool col_ok = col < G.N;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rit = wm * TM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const float v = acc[0][i][j][r];
          const float u = acc[NB - 1][i][j][r];
          if constexpr (!Tr::GROUP_K) {
            const int row = row0 + rit;
            if (col_ok && row < row_end) epilogue_rows<KIND>(args, G, row, col, v, u);
          } else {
            const int m = m0 + rit;
            if (col_ok && m < G.M) {
              float* outp = (float*)(KIND == KIND_DW13 && z ? args.out1 : args.out0);
              outp[(int64_t)e_loc * G.M * G.N + (int64_t)m * G.N + col] = v;
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

template <int BM, int BN, int BK, int WM, int WN, int KIND>
static hipError_t run_bf16(const GroupedGemmArgs& g, hipStream_t s) {
  const GemmGeom G = geom_of<KIND>(g.d, g.F);
  const int ntn = (G.N + BN - 1) / BN;
  int blocks;
  dim3 grid;
  if constexpr (Traits<KIND>::GROUP_K) {
    blocks = g.E_loc * ((G.M + BM - 1) / BM) * ntn;
    grid = dim3(blocks, KIND == KIND_DW13 ? 2 : 1);
  } else {
    // persistent over the device-side tile count; bounded by the worst case
    const int64_t worst = ((g.P_max + BM - 1) / BM + g.E_loc) * (int64_t)ntn;
    blocks = (int)(worst < 1024 ? worst : 1024);
    grid = dim3(blocks);
  }
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<BM, BN, BK, WM, WN, KIND>), grid, dim3(WM * WN * 64), 0, s, g);
  return hipGetLastError();
}

hipError_t gemm_bf16(int kind, const GroupedGemmArgs& g, hipStream_t s) {
  switch (kind) {
    case KIND_UP:   return run_bf16<128, 128, 64, 2, 2, KIND_UP>(g, s);
    case KIND_DOWN: return run_bf16<128, 128, 64, 2, 2, KIND_DOWN>(g, s);
    case KIND_DH:   return run_bf16<128, 128, 64, 2, 2, KIND_DH>(g, s);
    case KIND_DX:   return run_bf16<128, 128, 64, 2, 2, KIND_DX>(g, s);
    case KIND_DW2:  return run_bf16<128, 128, 64, 2, 2, KIND_DW2>(g, s);
    case KIND_DW13: return run_bf16<128, 128, 64, 2, 2, KIND_DW13>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mok
