// Router GEMM of the MoE layer and its gradients, on the 32x32x16 bf16 MFMA.
//
// The router scores every token against every expert before the top-k
// choice ([kucoin §01]: the router is the first of the steps around the
// expert FFNs); here the score is a dot product with a per-expert router
// vector: logits[t, e] = sum_i x[t, i] Wr[e, i], x and Wr bf16, fp32
// accumulation.  The backward pass returns dx = dlogits Wr and
// dWr = dlogits^T x in fp32.
//
// Forward: HBM-bound on x (T d 2 bytes; Wr is small and stays in L2).  One
// workgroup per 32 tokens x 128 experts, the K loop fed by direct-to-LDS
// copies five 64-wide stages deep; the expert tiles of one token tile run
// on the same XCD, so x is fetched from HBM once.
//
// Backward: the fp32 gradient enters the bf16 MFMA as two bf16 terms,
// g = hi + lo with hi = bf16(g), lo = bf16(g - hi) (residual below 2^-17 |g|);
// x and Wr are bf16 already, so each product is exact and only the fp32
// accumulation rounds.  dx writes T d 4 bytes and is bound by that write.
// dWr contracts over the T tokens: the tokens are cut into s slices whose
// partial [E, d] products are written into the dx buffer (before dx itself
// is computed) and summed in ascending slice order by a second pass.  Every
// output is accumulated in an order fixed by the shapes alone.
#include <algorithm>

#include "gemm_pipe.h"
#include "mok_device.h"
#include "mok_internal.h"
#include "route_token.h"
#include "router_gemm.h"

namespace mok {
namespace {

typedef short rg_i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) rg_i16x4_t rg_lds_i16x4_t;

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Fragment of columns [cb, cb + 32) of an LDS tile stored k-row by k-row
// (columns contiguous, `stride` bytes per k row): lane l gets the eight bf16
// of column cb + l % 32 at k = 16 kk + 8 (l / 32) + 0..7, through two
// transposing 4 x 4 reads.  In a group of 16 lanes, lane j addresses four
// consecutive columns of k row j / 4 and receives column j of the four rows.
__device__ __forceinline__ bf16x8_t read_tr(const uint8_t* base, int stride, int cb, int kk, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int kr = kk * 16 + 8 * (g >> 1) + (j >> 2);
  const int col = cb + 16 * (g & 1) + 4 * (j & 3);
  const uint8_t* p = base + kr * stride + col * 2;
  const rg_i16x4_t lo =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((rg_lds_i16x4_t*)(const __attribute__((address_space(3))) void*)p);
  const rg_i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (rg_lds_i16x4_t*)(const __attribute__((address_space(3))) void*)(p + 4 * stride));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Fragment of rows [rb, rb + 32) of an LDS tile stored row by row (k
// contiguous, `stride` bytes per row): lane l gets row rb + l % 32 at
// k = 16 kk + 8 (l / 32) + 0..7.
__device__ __forceinline__ bf16x8_t read_k(const uint8_t* base, int stride, int rb, int kk, int lane) {
  return *reinterpret_cast<const bf16x8_t*>(base + (rb + (lane & 31)) * stride + kk * 32 + (lane >> 5) * 16);
}

// Eight fp32 values as their bf16 high parts and bf16 residuals.
__device__ __forceinline__ void split8(const float (&v)[8], u32x4_t& hi, u32x4_t& lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const bf16_t b = f2bf(v[u]);
    h[u] = b;
    l[u] = f2bf(v[u] - bf2f(b));
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    hi[u] = h[2 * u] | (h[2 * u + 1] << 16);
    lo[u] = l[2 * u] | (l[2 * u + 1] << 16);
  }
}

// One thread's share of a staged K chunk: eight fp32 gradient values and 32
// bytes (sixteen bf16) of the other operand, held in registers while the
// previous chunk is multiplied.
struct Staged {
  float a[8];
  u32x4_t b0, b1;
};

// a[u] = ap[k0 + ac + u] where k0 + ac + u < alim, else 0; the sixteen bf16
// at bp + (k0 + br) ld where k0 + br < blim, else 0.  VEC: ap + k0 + ac is
// 16-byte aligned and alim a multiple of 4, so the eight floats come as two
// 16-byte loads, each wholly inside or wholly outside the limit.
template <bool VEC>
__device__ __forceinline__ Staged stage_load(const float* ap, int ac, int alim, const bf16_t* bp, int br,
                                             int64_t ld, int blim, int k0) {
  Staged v;
  if constexpr (VEC) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = k0 + ac + 4 * h;
      const f32x4_t q = k < alim ? *reinterpret_cast<const f32x4_t*>(ap + k) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u) v.a[4 * h + u] = q[u];
    }
  } else {
#pragma unroll
    for (int u = 0; u < 8; ++u) v.a[u] = k0 + ac + u < alim ? ap[k0 + ac + u] : 0.0f;
  }
  if (k0 + br < blim) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(bp + (int64_t)(k0 + br) * ld);
    v.b0 = p[0];
    v.b1 = p[1];
  } else {
    v.b0 = v.b1 = u32x4_t{0, 0, 0, 0};
  }
  return v;
}

// The gradient values as bf16 high parts and residuals at ah / al (16 bytes
// each), the other operand's 32 bytes at b.
__device__ __forceinline__ void stage_store(const Staged& v, uint8_t* ah, uint8_t* al, uint8_t* b) {
  u32x4_t h, l;
  split8(v.a, h, l);
  *reinterpret_cast<u32x4_t*>(ah) = h;
  *reinterpret_cast<u32x4_t*>(al) = l;
  *reinterpret_cast<u32x4_t*>(b) = v.b0;
  *reinterpret_cast<u32x4_t*>(b + 16) = v.b1;
}

// Store a 32 x 32 accumulator tile (rows r0.., columns c0..) of fp32 with
// row stride ld, keeping rows < nr and columns < nc.  Lanes 0..31 write 32
// consecutive floats of one row.
__device__ __forceinline__ void store_tile(float* out, int64_t ld, const f32x16_t& acc, int r0, int c0, int nr,
                                           int nc, int lane) {
  const int c = c0 + (lane & 31);
  if (c >= nc) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = r0 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
    if (row < nr) out[(int64_t)row * ld + c] = acc[r];
  }
}

// ------------------------------------------------------------------ forward
constexpr int kFwdBM = 32;   // tokens per tile
constexpr int kFwdBN = 128;  // experts per tile, 32 per wave
constexpr int kFwdBK = 64;   // K per stage: one 128-byte row piece
constexpr int kFwdNS = 5;    // stages in flight
constexpr int kFwdA = kFwdBM * kFwdBK * 2;
constexpr int kFwdStage = kFwdA + kFwdBN * kFwdBK * 2;
constexpr int kFwdCopies = kFwdStage / 1024 / 4;  // 16-byte copies per lane per stage
static_assert(kFwdA == 4 * 1024 && kFwdCopies == 5, "one A copy and four B copies per wave");

// One 32-token x 128-expert tile of the logits (tokens m0.., experts e0..):
// wave w returns experts e0 + 32 w .. as a 32 x 32 MFMA accumulator (lane l:
// expert column l % 32, token rows (r / 4) 8 + 4 (l / 32) + r % 4).  The K
// loop is fed by direct-to-LDS copies, kFwdNS stages deep; on return every
// copy has landed and every wave has passed the barrier after its last read
// of the arena.
__device__ __forceinline__ f32x16_t logits_tile(const bf16_t* __restrict__ x, const bf16_t* __restrict__ Wr, int d,
                                                int m0, int e0, int mrows, int erows, uint8_t* arena) {
  const int lane = lane_id(), wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // rows past the token / expert count read as zero
  const i32x4_t rsA = make_rsrc(x + (int64_t)m0 * d, (uint32_t)(mrows * d * 2));
  const i32x4_t rsB = make_rsrc(Wr + (int64_t)e0 * d, (uint32_t)(erows * d * 2));
  // Copy q of a wave fills 1 KB of the stage: lane i lands at slot 64 c + i
  // (row slot / 8, physical chunk slot % 8) with c = wid for the A copy and
  // 4 + 4 q' + wid for B copy q'; the swizzle is its own inverse.
  uint32_t offA, offB[4];
  {
    const int r = wid * 8 + (lane >> 3);
    offA = (uint32_t)(r * d * 2 + swz_k<kFwdBK>(r, lane & 7) * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rb = (q * 4 + wid) * 8 + (lane >> 3);
      offB[q] = (uint32_t)(rb * d * 2 + swz_k<kFwdBK>(rb, lane & 7) * 16);
    }
  }
  const int nk = d / kFwdBK;
  auto issue = [&](int s) {
    uint8_t* st = arena + (s % kFwdNS) * kFwdStage;
    const uint32_t soff = (uint32_t)(s * kFwdBK * 2);
    dma_b128(rsA, lds_addr(st + wid * 1024), offA, soff);
#pragma unroll
    for (int q = 0; q < 4; ++q) dma_b128(rsB, lds_addr(st + kFwdA + (q * 4 + wid) * 1024), offB[q], soff);
  };
  for (int s = 0; s < kFwdNS && s < nk; ++s) issue(s);

  f32x16_t acc = {};
  for (int s = 0; s < nk; ++s) {
    // stage s has landed once at most `later` younger stages are in flight
    wait_stages<kFwdCopies, kFwdNS - 1>(min(nk - 1 - s, kFwdNS - 1));
    const uint8_t* st = arena + (s % kFwdNS) * kFwdStage;
    bf16x8_t fa[4], fb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ra = lane & 31, rb = wid * 32 + (lane & 31), c = kk * 2 + (lane >> 5);
      fa[kk] = *reinterpret_cast<const bf16x8_t*>(st + ra * 128 + swz_k<kFwdBK>(ra, c) * 16);
      fb[kk] = *reinterpret_cast<const bf16x8_t*>(st + kFwdA + rb * 128 + swz_k<kFwdBK>(rb, c) * 16);
    }
    lds_barrier();  // every wave has read this buffer: it may be refilled
    if (s + kFwdNS < nk) issue(s + kFwdNS);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = mfma(fa[kk], fb[kk], acc);
  }
  return acc;
}

// Grid: 8 * ceil(nT / 8) * nE workgroups.  Workgroup b runs on XCD b % 8;
// the nE expert tiles of a token tile take consecutive slots of one XCD.
__global__ __launch_bounds__(256) void router_logits_kernel(const bf16_t* __restrict__ x,
                                                            const bf16_t* __restrict__ Wr, int T, int d, int E,
                                                            int nT, int nE, float* __restrict__ logits) {
  __shared__ __attribute__((aligned(1024))) uint8_t arena[kFwdNS * kFwdStage];
  const int b = blockIdx.x;
  const int slot = b >> 3;
  const int tt = (slot / nE) * 8 + (b & 7), et = slot % nE;
  if (tt >= nT) return;
  const int lane = lane_id(), wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m0 = tt * kFwdBM, e0 = et * kFwdBN;
  const int mrows = min(kFwdBM, T - m0), erows = min(kFwdBN, E - e0);
  const f32x16_t acc = logits_tile(x, Wr, d, m0, e0, mrows, erows, arena);
  store_tile(logits + (int64_t)m0 * E + e0, E, acc, 0, wid * 32, mrows, erows, lane);
}

// The router GEMM with the router step fused behind it, for E <= 128 (one
// expert tile holds every logit of its 32 tokens): the tile's logits go to
// `logits` (for the backward) and to LDS, where each wave routes every
// fourth token of the tile (route_token: the same top-k, gates and lse as
// the router kernel on those logits, bit for bit).  Grid: 8 * ceil(nT / 8).
template <int EPL, bool SIGM, bool RENORM>
__global__ __launch_bounds__(256) void router_fused_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ Wr,
                                                           int T, int d, int E, int k, int nT,
                                                           float* __restrict__ logits, int32_t* __restrict__ idx_out,
                                                           float* __restrict__ gate_out,
                                                           int32_t* __restrict__ idx_saved,
                                                           float* __restrict__ gate_saved, float* __restrict__ lse,
                                                           int32_t* __restrict__ status) {
  __shared__ __attribute__((aligned(1024))) uint8_t arena[kFwdNS * kFwdStage];
  static_assert(kFwdBM * kFwdBN * 4 + 4 * kRouterMaxK * 4 <= kFwdNS * kFwdStage, "logits and gates fit the arena");
  const int b = blockIdx.x;
  const int tt = (b >> 3) * 8 + (b & 7);
  if (tt >= nT) return;
  const int lane = lane_id(), wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m0 = tt * kFwdBM;
  const int mrows = min(kFwdBM, T - m0);
  const f32x16_t acc = logits_tile(x, Wr, d, m0, 0, mrows, E, arena);
  store_tile(logits + (int64_t)m0 * E, E, acc, 0, wid * 32, mrows, E, lane);
  lds_barrier();
  float* lg = reinterpret_cast<float*>(arena);  // [mrows][E]
  {
    const int c = wid * 32 + (lane & 31);
    if (c < E)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (row < mrows) lg[row * E + c] = acc[r];
      }
  }
  __syncthreads();
  float* graw = lg + kFwdBM * kFwdBN + (RENORM ? wid * kRouterMaxK : 0);  // this wave's raw gates
  for (int t = wid; t < mrows; t += 4)
    route_token<EPL, SIGM, RENORM>(lg + t * E, m0 + t, E, k, idx_out, gate_out, idx_saved, gate_saved, lse, status,
                                   graw);
}

// Both backward kernels stream K in chunks of 32 through one LDS buffer,
// with the next two chunks held in registers while a chunk is multiplied.
constexpr int kBK = 32;
constexpr int kKStride = kBK * 2 + 16;  // bytes per k-contiguous row (80: 16 rows hit distinct banks)

// Chunk v into LDS once every wave has finished with the previous one.
__device__ __forceinline__ void stage_chunk(const Staged& v, uint8_t* ah, uint8_t* al, uint8_t* b) {
  __syncthreads();
  stage_store(v, ah, al, b);
  __syncthreads();
}

// --------------------------------------------------------------- dx = g Wr
// Tile 64 tokens x 128 columns of d, K = experts.  Waves 2 x 2: rows 32 wm..,
// columns 64 wn.. (two 32-wide MFMA tiles).
constexpr int kDxBM = 64, kDxBN = 128;
constexpr int kDxBStride = kDxBN * 2 + 64;  // bytes per k row of the 128 columns (320: conflict-free transposing reads)

__device__ __forceinline__ void dx_mma(f32x16_t (&acc)[2], const uint8_t* ahi, const uint8_t* alo, const uint8_t* bs,
                                       int wm, int wn, int lane) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const bf16x8_t fh = read_k(ahi, kKStride, wm * 32, kk, lane), fl = read_k(alo, kKStride, wm * 32, kk, lane);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const bf16x8_t fb = read_tr(bs, kDxBStride, wn * 64 + nt * 32, kk, lane);
      acc[nt] = mfma(fh, fb, acc[nt]);
      acc[nt] = mfma(fl, fb, acc[nt]);
    }
  }
}

template <bool VEC>
__global__ __launch_bounds__(256) void router_dx_kernel(const float* __restrict__ g, const bf16_t* __restrict__ Wr,
                                                        int T, int d, int E, float* __restrict__ dx) {
  __shared__ __attribute__((aligned(16))) uint8_t ahi[kDxBM * kKStride], alo[kDxBM * kKStride];
  __shared__ __attribute__((aligned(16))) uint8_t bs[kBK * kDxBStride];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, wm = wid & 1, wn = wid >> 1;
  const int m0 = blockIdx.x * kDxBM, n0 = blockIdx.y * kDxBN;
  // staging: A rows tid / 4, eight experts from 8 (tid % 4); B k row tid / 8, sixteen columns from 16 (tid % 8)
  const int ar = tid >> 2, ac = (tid & 3) * 8, br = tid >> 3, bc = (tid & 7) * 16;
  const float* gp = g + (int64_t)(m0 + ar) * E;
  const bf16_t* wp = Wr + n0 + bc;
  const int alim = m0 + ar < T ? E : 0, blim = n0 + bc < d ? E : 0;
  uint8_t *sah = ahi + ar * kKStride + ac * 2, *sal = alo + ar * kKStride + ac * 2, *sb = bs + br * kDxBStride + bc * 2;
  f32x16_t acc[2] = {};
  Staged v0 = stage_load<VEC>(gp, ac, alim, wp, br, d, blim, 0), v1;
  if (kBK < E) v1 = stage_load<VEC>(gp, ac, alim, wp, br, d, blim, kBK);
  for (int k0 = 0; k0 < E; k0 += 2 * kBK) {
    stage_chunk(v0, sah, sal, sb);
    if (k0 + 2 * kBK < E) v0 = stage_load<VEC>(gp, ac, alim, wp, br, d, blim, k0 + 2 * kBK);
    dx_mma(acc, ahi, alo, bs, wm, wn, lane);
    if (k0 + kBK >= E) break;
    stage_chunk(v1, sah, sal, sb);
    if (k0 + 3 * kBK < E) v1 = stage_load<VEC>(gp, ac, alim, wp, br, d, blim, k0 + 3 * kBK);
    dx_mma(acc, ahi, alo, bs, wm, wn, lane);
  }
  const int nr = min(kDxBM, T - m0), nc = min(kDxBN, d - n0);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
    store_tile(dx + (int64_t)m0 * d + n0, d, acc[nt], wm * 32, wn * 64 + nt * 32, nr, nc, lane);
}

// ------------------------------------------------------ dWr slices = g^T x
// Tile 64 experts x 128 columns of d over the tokens [t0, t1) of slice
// blockIdx.z, K chunks of 32 tokens.  Waves 2 x 2 as in dx.  The output is
// slice z's [E, d] partial (or dWr itself when there is one slice).
constexpr int kDwBM = 64, kDwBN = 128;
constexpr int kDwAStride = kDwBM * 2 + 64;  // 192 bytes per token row of 64 experts
constexpr int kDwBStride = kDwBN * 2 + 64;  // 320 bytes per token row of 128 columns

__device__ __forceinline__ void dw_mma(f32x16_t (&acc)[2], const uint8_t* ghi, const uint8_t* glo, const uint8_t* xs,
                                       int wm, int wn, int lane) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const bf16x8_t fh = read_tr(ghi, kDwAStride, wm * 32, kk, lane), fl = read_tr(glo, kDwAStride, wm * 32, kk, lane);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const bf16x8_t fb = read_tr(xs, kDwBStride, wn * 64 + nt * 32, kk, lane);
      acc[nt] = mfma(fh, fb, acc[nt]);
      acc[nt] = mfma(fl, fb, acc[nt]);
    }
  }
}

// Token row k0 + r of a chunk: eight gradient values from expert e0 + ac
// (those below E) and sixteen columns of x from n0 + bc.
template <bool VEC>
__device__ __forceinline__ Staged dw_load(const float* g, const bf16_t* x, int64_t d, int E, int e0, int n0, int r,
                                          int ac, int bc, bool bcol, int t1, int k0) {
  const int t = k0 + r;
  const bool trow = t < t1;
  return stage_load<VEC>(g + (int64_t)t * E + e0, ac, trow ? E - e0 : 0, x + (int64_t)t * d + n0 + bc, 0, 0,
                         (trow && bcol) ? 1 : 0, 0);
}

template <bool VEC>
__global__ __launch_bounds__(256) void router_dw_kernel(const float* __restrict__ g, const bf16_t* __restrict__ x,
                                                        int T, int d, int E, int tslice,
                                                        float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint8_t ghi[kBK * kDwAStride], glo[kBK * kDwAStride];
  __shared__ __attribute__((aligned(16))) uint8_t xs[kBK * kDwBStride];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, wm = wid & 1, wn = wid >> 1;
  const int e0 = blockIdx.x * kDwBM, n0 = blockIdx.y * kDwBN;
  const int t0 = blockIdx.z * tslice, t1 = min(T, t0 + tslice);
  // staging: token row tid / 8 of the chunk; eight experts from 8 (tid % 8),
  // sixteen columns from 16 (tid % 8)
  const int r = tid >> 3, ac = (tid & 7) * 8, bc = (tid & 7) * 16;
  const bool bcol = n0 + bc < d;
  uint8_t *sgh = ghi + r * kDwAStride + ac * 2, *sgl = glo + r * kDwAStride + ac * 2, *sx = xs + r * kDwBStride + bc * 2;
  f32x16_t acc[2] = {};
  Staged v0 = dw_load<VEC>(g, x, d, E, e0, n0, r, ac, bc, bcol, t1, t0), v1;
  if (t0 + kBK < t1) v1 = dw_load<VEC>(g, x, d, E, e0, n0, r, ac, bc, bcol, t1, t0 + kBK);
  for (int k0 = t0; k0 < t1; k0 += 2 * kBK) {
    stage_chunk(v0, sgh, sgl, sx);
    if (k0 + 2 * kBK < t1) v0 = dw_load<VEC>(g, x, d, E, e0, n0, r, ac, bc, bcol, t1, k0 + 2 * kBK);
    dw_mma(acc, ghi, glo, xs, wm, wn, lane);
    if (k0 + kBK >= t1) break;
    stage_chunk(v1, sgh, sgl, sx);
    if (k0 + 3 * kBK < t1) v1 = dw_load<VEC>(g, x, d, E, e0, n0, r, ac, bc, bcol, t1, k0 + 3 * kBK);
    dw_mma(acc, ghi, glo, xs, wm, wn, lane);
  }
  float* out = part + (int64_t)blockIdx.z * E * d + (int64_t)e0 * d + n0;
  const int nr = min(kDwBM, E - e0), nc = min(kDwBN, d - n0);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) store_tile(out, d, acc[nt], wm * 32, wn * 64 + nt * 32, nr, nc, lane);
}

// dWr = sum over the slices in ascending order, four floats per thread.
__global__ __launch_bounds__(256) void router_dw_reduce_kernel(const f32x4_t* __restrict__ part, int64_t n4,
                                                               int splits, f32x4_t* __restrict__ dWr) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  f32x4_t s = part[i];
  for (int z = 1; z < splits; ++z) s += part[(int64_t)z * n4 + i];
  dWr[i] = s;
}

inline int cdiv(int a, int b) { return (a + b - 1) / b; }

}  // namespace

int router_dw_splits(int T, int d, int E) {
  const int tiles = cdiv(E, kDwBM) * cdiv(d, kDwBN);
  int s = cdiv(512, tiles);       // about two workgroups per compute unit
  s = std::min(s, 64);
  s = std::min(s, T / E);         // the slices' partials must fit in dx [T, d]
  s = std::min(s, cdiv(T, kBK));  // at least one chunk of tokens per slice
  return std::max(s, 1);
}

hipError_t launch_router_logits(const void* x, const void* Wr, int T, int d, int E, float* logits, hipStream_t s) {
  const int nT = cdiv(T, kFwdBM), nE = cdiv(E, kFwdBN);
  const int grid = 8 * cdiv(nT, 8) * nE;
  hipLaunchKernelGGL(router_logits_kernel, dim3(grid), dim3(256), 0, s, (const bf16_t*)x, (const bf16_t*)Wr, T, d,
                     E, nT, nE, logits);
  return hipGetLastError();
}

hipError_t launch_router_fused(const void* x, const void* Wr, int T, int d, int E, int k, int gating, float* logits,
                               int32_t* idx_out, float* gate_out, int32_t* idx_saved, float* gate_saved, float* lse,
                               int32_t* status, hipStream_t s) {
  if (E > kFwdBN || E < 1 || k < 1 || k > E) return hipErrorInvalidValue;
  const int nT = cdiv(T, kFwdBM);
  if (nT == 0) return hipSuccess;
  const dim3 g(8 * cdiv(nT, 8)), blk(256);
  const bool sg = gating & kGateSigmoid, rn = gating & kGateRenorm;
#define MOK_FUSED(EPLV, SG, RN)                                                                                      \
  hipLaunchKernelGGL((router_fused_kernel<EPLV, SG, RN>), g, blk, 0, s, (const bf16_t*)x, (const bf16_t*)Wr, T, d, E, k, \
                     nT, logits, idx_out, gate_out, idx_saved, gate_saved, lse, status)
#define MOK_FUSED_E(SG, RN)        \
  if (E <= 64) MOK_FUSED(1, SG, RN); \
  else MOK_FUSED(2, SG, RN);
  if (!sg && !rn) { MOK_FUSED_E(false, false) }
  else if (sg && !rn) { MOK_FUSED_E(true, false) }
  else if (!sg && rn) { MOK_FUSED_E(false, true) }
  else { MOK_FUSED_E(true, true) }
#undef MOK_FUSED_E
#undef MOK_FUSED
  return hipGetLastError();
}

hipError_t launch_router_logits_backward(const void* x, const void* Wr, const float* dlogits, int T, int d, int E,
                                         float* dx, float* dWr, hipStream_t s) {
  const int splits = router_dw_splits(T, d, E);
  const int slice = std::max(cdiv(cdiv(T, splits), kBK), 1) * kBK;
  const int nz = std::max(cdiv(T, slice), 1);  // T = 0: one slice of nothing, dWr = 0
  float* part = nz > 1 ? dx : dWr;
  // 16-byte gradient loads when every row starts 16-byte aligned
  const bool vec = E % 4 == 0 && ((uintptr_t)dlogits & 15) == 0;
  const dim3 gw(cdiv(E, kDwBM), cdiv(d, kDwBN), nz);
  if (vec) hipLaunchKernelGGL(router_dw_kernel<true>, gw, dim3(256), 0, s, dlogits, (const bf16_t*)x, T, d, E, slice, part);
  else hipLaunchKernelGGL(router_dw_kernel<false>, gw, dim3(256), 0, s, dlogits, (const bf16_t*)x, T, d, E, slice, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nz > 1) {
    const int64_t n4 = (int64_t)E * d / 4;
    hipLaunchKernelGGL(router_dw_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                       (const f32x4_t*)part, n4, nz, (f32x4_t*)dWr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (T == 0) return hipSuccess;
  const dim3 gx(cdiv(T, kDxBM), cdiv(d, kDxBN));
  if (vec) hipLaunchKernelGGL(router_dx_kernel<true>, gx, dim3(256), 0, s, dlogits, (const bf16_t*)Wr, T, d, E, dx);
  else hipLaunchKernelGGL(router_dx_kernel<false>, gx, dim3(256), 0, s, dlogits, (const bf16_t*)Wr, T, d, E, dx);
  return hipGetLastError();
}

}  // namespace mok
