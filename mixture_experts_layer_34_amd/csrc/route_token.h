// Router softmax + stable top-k of one token by one wave, shared by the
// router kernels (route_sort.hip) and the router GEMM's fused form
// (router_gemm.hip), so that every path takes the same decisions bit for bit.
//
// Selection order: logit descending, expert index ascending on ties, comparing
// the raw fp32 logits (kucoin.com, "Cursor's MoK réalise une amélioration des
// performances de 2,37x sur NVIDIA GB300 NVL72", section 01: the router picks
// several experts per token).
#pragma once
#include "mok_device.h"

namespace mok {

// One wave per token; lane l holds logits e = l + 64 i.  k rounds of a wave
// arg-max under the (value desc, index asc) order.  Gates: the softmax
// probability of the chosen expert, or its sigmoid (SIGM); with RENORM each
// is divided by their sum over the k chosen experts (slot order, fp32).
constexpr int kRouterMaxK = 1024;  // k <= E <= 1024
// One token's routing by one wave: top-k of its raw logits `row` (E fp32
// values, global memory or LDS), gates, lse; outputs at token t.  graw: this
// wave's k floats of LDS (renormalised gates only).
template <int EPL, bool SIGM, bool RENORM>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int t, int E, int k,
                                            int32_t* __restrict__ idx_out, float* __restrict__ gate_out,
                                            int32_t* __restrict__ idx_saved, float* __restrict__ gate_saved,
                                            float* __restrict__ lse_out, int32_t* __restrict__ status,
                                            float* graw) {
  const int lane = lane_id();
  float v[EPL];
  float m = -INFINITY;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -INFINITY;
    // logits must be finite: a NaN or an infinity is reported, and a NaN
    // is ranked as -inf so that the k chosen indices stay in [0, E)
    if (e < E && !isfinite(v[i])) {
      bad = true;
      if (v[i] != v[i]) v[i] = -INFINITY;
    }
    m = fmaxf(m, v[i]);
  }
  if (__ballot(bad) != 0 && lane == 0) report(status, kCheckLogits);
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    int e = lane + 64 * i;
    if (e < E) s += expf(v[i] - m);
  }
  s = wave_sum(s);
  const float inv_s = 1.0f / s;
  // Selection key of each candidate: the logit mapped to an order-preserving
  // unsigned code (with -0 taken as +0, so that equal values tie) in the high
  // word, 2^32 - 1 - e in the low word: the largest key is the largest
  // value, lowest index first.  A chosen or absent candidate has key 0, below
  // every real key (-inf maps to 0x007fffff).
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    uint32_t u = __float_as_uint(v[i]);
    if ((u << 1) == 0) u = 0;
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    key[i] = e < E ? ((uint64_t)ord << 32) | (0xFFFFFFFFu - (uint32_t)e) : 0ull;
  }
  float gsum = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int be = (int)(0xFFFFFFFFu - (uint32_t)best);
    const uint32_t ord = (uint32_t)(best >> 32);
    const float bv = __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + 64 * i == be) key[i] = 0ull;
    if (lane == 0) {
      const float g = SIGM ? 1.0f / (1.0f + expf(-bv)) : expf(bv - m) * inv_s;
      idx_out[(int64_t)t * k + j] = be;
      idx_saved[(int64_t)t * k + j] = be;
      if constexpr (RENORM) {
        graw[j] = g;
        gsum += g;
      } else {
        gate_out[(int64_t)t * k + j] = g;
        gate_saved[(int64_t)t * k + j] = g;
      }
    }
  }
  if (lane == 0) {
    lse_out[t] = m + logf(s);
    if constexpr (RENORM) {
      for (int j = 0; j < k; ++j) {
        const float g = graw[j] / gsum;
        gate_out[(int64_t)t * k + j] = g;
        gate_saved[(int64_t)t * k + j] = g;
      }
    }
  }
}

}  // namespace mok
