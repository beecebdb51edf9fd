// Host-side launchers of the router GEMM kernels (logits = x Wr^T and its two
// gradients).  Internal to libmok; the public interface is include/mok.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mok {

// Number of token slices the weight gradient dWr = dlogits^T x is split into:
// each slice's partial [E, d] product lands in the dx buffer (so s * E <= T)
// and a second pass sums the slices in ascending order.  Depends on the
// shapes only, so the result is run-to-run identical.
int router_dw_splits(int T, int d, int E);

// x bf16 [T, d], Wr bf16 [E, d], logits fp32 [T, E].
hipError_t launch_router_logits(const void* x, const void* Wr, int T, int d, int E, float* logits, hipStream_t s);

constexpr int kRouterFusedMaxE = 128;  // experts of one router GEMM tile

// The same logits with the router step fused behind them (E <= 128, one
// expert tile per 32 tokens): logits written as by launch_router_logits, and
// idx / gates / lse as launch_router_topk writes them from those logits.
// gating: kGateSigmoid / kGateRenorm bits.  hipErrorInvalidValue for E > 128.
hipError_t launch_router_fused(const void* x, const void* Wr, int T, int d, int E, int k, int gating, float* logits,
                               int32_t* idx_out, float* gate_out, int32_t* idx_saved, float* gate_saved, float* lse,
                               int32_t* status, hipStream_t s);

// dlogits fp32 [T, E]; dx fp32 [T, d] (also the scratch of the dWr slices),
// dWr fp32 [E, d].
hipError_t launch_router_logits_backward(const void* x, const void* Wr, const float* dlogits, int T, int d, int E,
                                         float* dx, float* dWr, hipStream_t s);

}  // namespace mok
