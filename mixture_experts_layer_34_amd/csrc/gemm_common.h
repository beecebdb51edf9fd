// Geometry of the six expert-grouped GEMMs of the MoE layer (shared by the
// BF16 MFMA, MXFP8 scaled-MFMA and fp32 kernels).
#pragma once
#include "mok_internal.h"

namespace mok {

enum GemmKind { KIND_UP = 0, KIND_DOWN = 1, KIND_DH = 2, KIND_DX = 3, KIND_DW2 = 4, KIND_DW13 = 5 };

// A_MN / B_MN: the operand is stored with M (resp. N) contiguous and K strided
// (otherwise K-contiguous).  NB: number of B matrices (UP pairs W1 with W3).
// GROUP_K: the expert's rows are the K dimension (weight gradients).
template <int KIND> struct Traits;
template <> struct Traits<KIND_UP>   { static constexpr bool A_MN = false, B_MN = false, GROUP_K = false; static constexpr int NB = 2; };
template <> struct Traits<KIND_DOWN> { static constexpr bool A_MN = false, B_MN = false, GROUP_K = false; static constexpr int NB = 1; };
template <> struct Traits<KIND_DH>   { static constexpr bool A_MN = false, B_MN = true,  GROUP_K = false; static constexpr int NB = 1; };
template <> struct Traits<KIND_DX>   { static constexpr bool A_MN = false, B_MN = true,  GROUP_K = false; static constexpr int NB = 1; };
template <> struct Traits<KIND_DW2>  { static constexpr bool A_MN = true,  B_MN = true,  GROUP_K = true;  static constexpr int NB = 1; };
template <> struct Traits<KIND_DW13> { static constexpr bool A_MN = true,  B_MN = true,  GROUP_K = true;  static constexpr int NB = 1; };

struct GemmGeom {
  int M, N, K;            // M only for GROUP_K kinds (K for those = expert rows)
  int64_t lda, ldb;       // element strides of the K (or MN) rows
  int64_t b_estride;      // elements between consecutive experts' weights
  int ksplit;             // DX: K rows below ksplit come from B0, the rest from B1
};

template <int KIND>
__host__ __device__ inline GemmGeom geom_of(int d, int F) {
  GemmGeom g{};
  switch (KIND) {
    case KIND_UP:   g.N = F; g.K = d; g.lda = d; g.ldb = d; g.b_estride = (int64_t)F * d; g.ksplit = d; break;
    case KIND_DOWN: g.N = d; g.K = F; g.lda = F; g.ldb = F; g.b_estride = (int64_t)d * F; g.ksplit = F; break;
    case KIND_DH:   g.N = F; g.K = d; g.lda = d; g.ldb = F; g.b_estride = (int64_t)d * F; g.ksplit = d; break;
    case KIND_DX:   g.N = d; g.K = 2 * F; g.lda = 2 * F; g.ldb = d; g.b_estride = (int64_t)F * d; g.ksplit = F; break;
    case KIND_DW2:  g.M = d; g.N = F; g.lda = d; g.ldb = F; break;
    case KIND_DW13: g.M = F; g.N = d; g.lda = 2 * F; g.ldb = d; break;
  }
  return g;
}

}  // namespace mok
