// Router softmax + stable top-k, and the counting sort that lays token-expert
// pairs out expert-contiguously.
//
// The router picks several experts per token at every step, and before any
// token moves the system counts the tokens of each expert and decides where
// each one lands, keeping one expert's tokens together for the grouped GEMM
// (kucoin.com, "Cursor's MoK réalise une amélioration des performances de
// 2,37x sur NVIDIA GB300 NVL72", section 01).  The receiver chooses the local
// placement itself (same page, section 02, pull dispatch).
//
// Selection order: logit descending, expert index ascending on ties, comparing
// the raw fp32 logits.  Placement is stable: within one expert, rows ascend by
// pair id p = t*k + j.  Both are integer-exact and run-to-run identical.
#include "mok_device.h"
#include "mok_internal.h"
#include "route_token.h"

namespace mok {

// ------------------------------------------------------------------ router
// One wave per token (route_token.h), grid-stride over the tokens.
template <int EPL, bool SIGM, bool RENORM>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits, int T,
                                                          int E, int k, int32_t* __restrict__ idx_out,
                                                          float* __restrict__ gate_out,
                                                          int32_t* __restrict__ idx_saved,
                                                          float* __restrict__ gate_saved,
                                                          float* __restrict__ lse_out,
                                                          int32_t* __restrict__ status) {
  __shared__ float renorm_buf[RENORM ? 4 * kRouterMaxK : 1];
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  float* graw = RENORM ? renorm_buf + (threadIdx.x >> 6) * kRouterMaxK : renorm_buf;  // this wave's raw gates
  for (int t = wave; t < T; t += nwaves)
    route_token<EPL, SIGM, RENORM>(logits + (int64_t)t * E, t, E, k, idx_out, gate_out, idx_saved, gate_saved, lse_out,
                                   status, graw);
}

template <bool SIGM, bool RENORM>
static void launch_router_variant(dim3 g, dim3 b, hipStream_t s, const float* logits, int T, int E, int k,
                                  int32_t* idx_out, float* gate_out, int32_t* idx_saved, float* gate_saved,
                                  float* lse, int32_t* status) {
#define MOK_ROUTER(EPLV)                                                                                   \
  hipLaunchKernelGGL((router_topk_kernel<EPLV, SIGM, RENORM>), g, b, 0, s, logits, T, E, k, idx_out, gate_out, \
                     idx_saved, gate_saved, lse, status)
  if (E <= 64) MOK_ROUTER(1);
  else if (E <= 128) MOK_ROUTER(2);
  else if (E <= 256) MOK_ROUTER(4);
  else if (E <= 512) MOK_ROUTER(8);
  else MOK_ROUTER(16);
#undef MOK_ROUTER
}

hipError_t launch_router_topk(const float* logits, int T, int E, int k, int gating, int32_t* idx_out,
                              float* gate_out, int32_t* idx_saved, float* gate_saved, float* lse,
                              int32_t* status, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int blocks = (T + 3) / 4;
  if (blocks > 8192) blocks = 8192;
  const dim3 g(blocks), b(256);
  switch (gating & (kGateSigmoid | kGateRenorm)) {
    case 0: launch_router_variant<false, false>(g, b, s, logits, T, E, k, idx_out, gate_out, idx_saved, gate_saved, lse, status); break;
    case kGateSigmoid: launch_router_variant<true, false>(g, b, s, logits, T, E, k, idx_out, gate_out, idx_saved, gate_saved, lse, status); break;
    case kGateRenorm: launch_router_variant<false, true>(g, b, s, logits, T, E, k, idx_out, gate_out, idx_saved, gate_saved, lse, status); break;
    default: launch_router_variant<true, true>(g, b, s, logits, T, E, k, idx_out, gate_out, idx_saved, gate_saved, lse, status); break;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ status word
// Clears the status word (MOK_OK, no failed checks) at the start of a call.
__global__ void status_reset_kernel(int32_t* status) {
  if (threadIdx.x < 2) status[threadIdx.x] = 0;
}

hipError_t launch_status_reset(int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(status_reset_kernel, dim3(1), dim3(64), 0, s, status);
  return hipGetLastError();
}

// ------------------------------------------------------------------ counting sort
// Lanes of a wave holding the same expert: AND over the expert-id bits of the
// ballot of each bit (or of its complement), restricted to valid lanes.
__device__ __forceinline__ uint64_t peer_mask(int e, bool valid, int nbits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    bool bit = (e >> b) & 1;
    uint64_t bm = __ballot(bit);
    m &= bit ? bm : ~bm;
  }
  return m;
}

// A wave's chunk of expert ids, all loaded at once (pair base + 64 i + lane in
// ev[i]) so that the walk over the chunk waits for memory only once; -1 past
// the end.
constexpr int kChunkIters = kSortChunk / 64;
__device__ __forceinline__ void load_chunk(const int32_t* __restrict__ idx, int64_t npairs, int64_t base,
                                           int lane, int (&ev)[kChunkIters]) {
#pragma unroll
  for (int it = 0; it < kChunkIters; ++it) {
    const int64_t p = base + it * 64 + lane;
    ev[it] = p < npairs ? idx[p] : -1;
  }
}

// Pass 1: per-chunk expert histogram.  One wave per chunk of kSortChunk pairs;
// the lowest lane of each group of equal experts adds the group's size.
__global__ __launch_bounds__(256) void sort_hist_kernel(const int32_t* __restrict__ idx, int64_t npairs,
                                                        int E, int eb, int ee, int nbits, int nchunks,
                                                        int32_t* __restrict__ chunk_counts) {
  extern __shared__ int32_t hist_smem[];
  const int w = threadIdx.x >> 6, lane = lane_id();
  const int c = blockIdx.x * 4 + w;
  int32_t* hist = hist_smem + w * E;
  for (int e = lane; e < E; e += 64) hist[e] = 0;
  __syncthreads();
  if (c < nchunks) {
    int ev[kChunkIters];
    load_chunk(idx, npairs, (int64_t)c * kSortChunk, lane, ev);
#pragma unroll
    for (int it = 0; it < kChunkIters; ++it) {
      const int e = ev[it];
      bool valid = e >= eb && e < ee;
      uint64_t m = peer_mask(e, valid, nbits);
      if (valid && lane == __ffsll((unsigned long long)m) - 1) hist[e] += __popcll(m);
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
  if (c < nchunks)
    for (int e = lane; e < E; e += 64) chunk_counts[(int64_t)c * E + e] = hist[e];
}

// Pass 2: one block.  The chunks of each expert are split among G = 1024 / E
// threads (thread g * E + e takes the g-th contiguous share of chunks); the
// shares' sums give each expert's total and each share's starting count.  The
// block scans the totals over experts (offsets), each share then writes its
// chunk bases, and the row-tile prefix of the local experts is written for
// each tile height.
// Offsets, counts, tile prefixes and the heaviest-first weight-gradient
// schedule of the experts, from each expert's pair count: called by every
// thread of a 1024-thread block with run = the count of expert threadIdx.x
// (0 past E).  Writes s_offE[e] (the expert's first row, visible to the
// whole block on return) and returns it.
__device__ int scan_and_schedule(int run, int E, int eb, int ee, int32_t* __restrict__ counts_out,
                                 int32_t* __restrict__ offsets_out, int32_t* __restrict__ offsets_saved,
                                 int32_t* __restrict__ tile_prefix, int32_t* __restrict__ expert_order,
                                 int32_t* s_offE) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t s_cnt[1024];
  __shared__ int32_t tsum[kNumTileBM][16];
  const int e = threadIdx.x;
  const int lane = lane_id(), w = threadIdx.x >> 6;
  // exclusive scan of run over e (1024 threads = 16 waves)
  int incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wsum[w] = incl;
  // tile counts of local expert i = e - eb for each tile height
  const int E_loc = ee - eb;
  const int i_loc = e - eb;
  int tinc[kNumTileBM];
#pragma unroll
  for (int b = 0; b < kNumTileBM; ++b) {
    int tc = (i_loc >= 0 && i_loc < E_loc) ? (run + kTileBM[b] - 1) / kTileBM[b] : 0;
    int x = tc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int u = __shfl_up(x, o, 64);
      if (lane >= o) x += u;
    }
    tinc[b] = x;
    if (lane == 63) tsum[b][w] = x;
  }
  __syncthreads();
  int wbase = 0;
  int tbase[kNumTileBM] = {};
  for (int q = 0; q < w; ++q) {
    wbase += wsum[q];
#pragma unroll
    for (int b = 0; b < kNumTileBM; ++b) tbase[b] += tsum[b][q];
  }
  const int off = wbase + incl - run;
  if (e < E) {
    counts_out[e] = run;
    offsets_out[e] = off;
    offsets_saved[e] = off;
    s_offE[e] = off;
    if (e == E - 1) {
      offsets_out[E] = off + run;
      offsets_saved[E] = off + run;
    }
  }
  // Weight-gradient schedule: local experts ranked by descending row count
  // (ties: lower index), with the prefix of their work in K stages of 32
  // rows plus 10 per tile (a tile's fixed set-up and epilogue cost about as
  // much as ten stages).  The weight-gradient GEMMs cut this heaviest-first
  // tile sequence into 8 runs of equal work, one per XCD.  Output: one
  // 16-byte record per rank r < E_loc, {local expert, first row, end row,
  // work of ranks 0 .. r-1}, and record E_loc = {0, 0, 0, total work}.
  __shared__ int32_t s_rank_e[1024], s_off[1024];
  if (i_loc >= 0 && i_loc < E_loc) {
    s_cnt[i_loc] = run;
    s_off[i_loc] = off;
  }
  __syncthreads();
  if (i_loc >= 0 && i_loc < E_loc) {
    int rank = 0;
    for (int q = 0; q < E_loc; ++q) {
      const int cq = s_cnt[q];
      rank += (cq > run || (cq == run && q < i_loc)) ? 1 : 0;
    }
    s_rank_e[rank] = i_loc;
  }
  __syncthreads();
  {
    // thread r: work of rank r, block-wide inclusive scan
    const int r = threadIdx.x;
    const int er = r < E_loc ? s_rank_e[r] : 0;
    const int wr = r < E_loc ? (s_cnt[er] + 31) / 32 + 10 : 0;
    int x = wr;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(x, o, 64);
      if (lane >= o) x += u;
    }
    __syncthreads();  // wsum is reused
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int base = 0;
    for (int q = 0; q < w; ++q) base += wsum[q];
    if (r < E_loc) {
      int32_t* rec = expert_order + 4 * r;
      rec[0] = er;
      rec[1] = s_off[er];
      rec[2] = s_off[er] + s_cnt[er];
      rec[3] = base + x - wr;
    }
    if (r == E_loc - 1 || (E_loc == 0 && r == 0)) {
      int32_t* rec = expert_order + 4 * E_loc;
      rec[0] = rec[1] = rec[2] = 0;
      rec[3] = E_loc ? base + x : 0;
    }
  }
  if (i_loc >= 0 && i_loc < E_loc) {
#pragma unroll
    for (int b = 0; b < kNumTileBM; ++b) {
      int inc = tbase[b] + tinc[b];
      int* tp = tile_prefix + b * (E_loc + 1);
      tp[i_loc + 1] = inc;
      if (i_loc == 0) tp[0] = 0;
    }
  }
  return off;
}

__global__ __launch_bounds__(1024) void sort_scan_kernel(const int32_t* __restrict__ chunk_counts,
                                                         int nchunks, int E, int eb, int ee,
                                                         int32_t* __restrict__ chunk_base,
                                                         int32_t* __restrict__ counts_out,
                                                         int32_t* __restrict__ offsets_out,
                                                         int32_t* __restrict__ offsets_saved,
                                                         int32_t* __restrict__ tile_prefix,
                                                         int32_t* __restrict__ expert_order) {
  __shared__ int32_t s_part[1024], s_offE[1024];
  const int e = threadIdx.x;
  // shares: thread (tg, te) = (threadIdx.x / E, threadIdx.x % E), tg < G
  const int G = 1024 / E;
  const int te = threadIdx.x % E, tg = threadIdx.x / E;
  const bool share = tg < G;
  const int c0 = share ? (int)((int64_t)nchunks * tg / G) : 0;
  const int c1 = share ? (int)((int64_t)nchunks * (tg + 1) / G) : 0;
  {
    int part = 0;
#pragma unroll 8
    for (int c = c0; c < c1; ++c) part += chunk_counts[(int64_t)c * E + te];
    if (share) s_part[threadIdx.x] = part;
  }
  __syncthreads();
  int run = 0;  // expert e's total
  if (e < E)
    for (int q = 0; q < G; ++q) run += s_part[q * E + e];
  const int off = scan_and_schedule(run, E, eb, ee, counts_out, offsets_out, offsets_saved, tile_prefix,
                                    expert_order, s_offE);
  (void)off;
  if (share) {
    // chunk bases of this share: the expert's first row, the counts of the
    // earlier shares, then a running sum over the share's chunks
    int r = s_offE[te];
    for (int q = 0; q < tg; ++q) r += s_part[q * E + te];
#pragma unroll 8
    for (int c = c0; c < c1; ++c) {
      const int v = chunk_counts[(int64_t)c * E + te];
      chunk_base[(int64_t)c * E + te] = r;
      r += v;
    }
  }
}

// Pass 3: stable placement.  Each wave re-walks its chunk in pair order with a
// running row per expert (in LDS) started at the chunk base; a pair's row is
// that running value plus its rank among the equal-expert lanes before it.
__global__ __launch_bounds__(256) void sort_scatter_kernel(const int32_t* __restrict__ idx, int64_t npairs,
                                                           int E, int eb, int ee, int nbits, int nchunks,
                                                           const int32_t* __restrict__ chunk_base,
                                                           int32_t* __restrict__ row_of_pair,
                                                           int32_t* __restrict__ pair_of_row) {
  extern __shared__ int32_t run_smem[];
  const int w = threadIdx.x >> 6, lane = lane_id();
  const int c = blockIdx.x * 4 + w;
  int32_t* run = run_smem + w * E;
  if (c < nchunks)
    for (int e = lane; e < E; e += 64) run[e] = chunk_base[(int64_t)c * E + e];
  __syncthreads();
  if (c >= nchunks) return;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t base = (int64_t)c * kSortChunk;
  int ev[kChunkIters];
  load_chunk(idx, npairs, base, lane, ev);
#pragma unroll
  for (int it = 0; it < kChunkIters; ++it) {
    const int64_t p = base + it * 64 + lane;
    const bool inb = p < npairs;
    const int e = ev[it];
    bool valid = e >= eb && e < ee;
    uint64_t m = peer_mask(e, valid, nbits);
    int row = -1;
    if (valid) row = run[e] + __popcll(m & lt);
    __builtin_amdgcn_wave_barrier();
    if (valid && lane == __ffsll((unsigned long long)m) - 1) run[e] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
    if (inb) row_of_pair[p] = row;
    if (valid) pair_of_row[row] = (int32_t)p;
  }
}

// ------------------------------------------------------------------ small-T path
// Router and counting sort in one workgroup of 1024 threads, for calls of at
// most kSmallTokens tokens and kSmallPairs token-expert pairs (a decode-style
// step): the status words
// are cleared, each of the 16 waves routes every 16th token (route_token, as
// the router kernel), then the block counts the local pairs per expert,
// scans them (scan_and_schedule, as the scan kernel) and places the pairs in
// chunks of 1024, stably: a pair's row is its expert's first row, plus the
// pairs of that expert in earlier chunks, in earlier waves of its chunk and in
// lower lanes of its wave.  The outputs are those of the router kernel and
// the three counting-sort kernels, bit for bit, in one launch instead of five.
template <int EPL, bool SIGM, bool RENORM>
__global__ __launch_bounds__(1024) void route_sort_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int eb, int ee, int nbits,
    int32_t* __restrict__ idx_out, float* __restrict__ gate_out, int32_t* __restrict__ idx_saved,
    float* __restrict__ gate_saved, float* __restrict__ lse_out, int32_t* __restrict__ counts_out,
    int32_t* __restrict__ offsets_out, int32_t* __restrict__ offsets_saved, int32_t* __restrict__ tile_prefix,
    int32_t* __restrict__ expert_order, int32_t* __restrict__ row_of_pair, int32_t* __restrict__ pair_of_row,
    int32_t* __restrict__ status) {
  // s_wcnt[w][e]: the pairs of expert e in wave w of the current chunk; while
  // the tokens are routed, wave w's row holds its raw gates (RENORM)
  __shared__ int32_t s_wcnt[16][1024];
  __shared__ int32_t s_hist[1024], s_base[1024], s_offE[1024];
  const int tid = threadIdx.x, w = tid >> 6, lane = lane_id();
  if (tid < 2) status[tid] = 0;
  __syncthreads();  // cleared before any check reports
  static_assert(kRouterMaxK <= 1024, "a wave's raw gates fit its row of s_wcnt");
  float* graw = reinterpret_cast<float*>(&s_wcnt[w][0]);
  for (int t = w; t < T; t += 16)
    route_token<EPL, SIGM, RENORM>(logits + (int64_t)t * E, t, E, k, idx_out, gate_out, idx_saved, gate_saved, lse_out,
                                   status, graw);
  if (tid < E) s_hist[tid] = 0;
  __syncthreads();  // the block's index writes are visible to the block
  const int npairs = T * k;
  for (int p = tid; p < npairs; p += 1024) {
    const int e = idx_saved[p];
    if (e >= eb && e < ee) atomicAdd(&s_hist[e], 1);
  }
  __syncthreads();
  const int run = tid < E ? s_hist[tid] : 0;
  scan_and_schedule(run, E, eb, ee, counts_out, offsets_out, offsets_saved, tile_prefix, expert_order, s_offE);
  if (tid < E) s_base[tid] = s_offE[tid];
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < npairs; c0 += 1024) {
    for (int e = lane; e < E; e += 64) s_wcnt[w][e] = 0;
    __syncthreads();  // s_wcnt cleared; s_base holds this chunk's first rows
    const int p = c0 + tid;
    const int e = p < npairs ? idx_saved[p] : -1;
    const bool valid = e >= eb && e < ee;
    const uint64_t m = peer_mask(e, valid, nbits);
    if (valid && lane == __ffsll((unsigned long long)m) - 1) s_wcnt[w][e] = __popcll(m);
    __syncthreads();
    int row = -1;
    if (valid) {
      row = s_base[e] + __popcll(m & lt);
      for (int q = 0; q < w; ++q) row += s_wcnt[q][e];
    }
    int chunk_total = 0;
    if (tid < E)
      for (int q = 0; q < 16; ++q) chunk_total += s_wcnt[q][tid];
    __syncthreads();  // s_base and s_wcnt read for this chunk
    if (tid < E) s_base[tid] += chunk_total;
    if (p < npairs) row_of_pair[p] = row;
    if (valid) pair_of_row[row] = p;
  }
}

template <bool SIGM, bool RENORM>
static void launch_small_variant(hipStream_t s, const float* logits, int T, int E, int k, int eb, int ee, int nbits,
                                 int32_t* idx_out, float* gate_out, int32_t* idx_saved, float* gate_saved,
                                 float* lse, int32_t* counts_out, int32_t* offsets_out, int32_t* offsets_saved,
                                 int32_t* tile_prefix, int32_t* expert_order, int32_t* row_of_pair,
                                 int32_t* pair_of_row, int32_t* status) {
#define MOK_SMALL(EPLV)                                                                                         \
  hipLaunchKernelGGL((route_sort_small_kernel<EPLV, SIGM, RENORM>), dim3(1), dim3(1024), 0, s, logits, T, E, k, eb, \
                     ee, nbits, idx_out, gate_out, idx_saved, gate_saved, lse, counts_out, offsets_out,          \
                     offsets_saved, tile_prefix, expert_order, row_of_pair, pair_of_row, status)
  if (E <= 64) MOK_SMALL(1);
  else if (E <= 128) MOK_SMALL(2);
  else if (E <= 256) MOK_SMALL(4);
  else if (E <= 512) MOK_SMALL(8);
  else MOK_SMALL(16);
#undef MOK_SMALL
}

hipError_t launch_route_sort_small(const float* logits, int T, int E, int k, int gating, int eb, int ee,
                                   int32_t* idx_out, float* gate_out, int32_t* idx_saved, float* gate_saved,
                                   float* lse, int32_t* counts_out, int32_t* offsets_out, int32_t* offsets_saved,
                                   int32_t* tile_prefix, int32_t* expert_order, int32_t* row_of_pair,
                                   int32_t* pair_of_row, int32_t* status, hipStream_t s) {
  if (T < 1 || T > kSmallTokens || (int64_t)T * k > kSmallPairs) return hipErrorInvalidValue;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  switch (gating & (kGateSigmoid | kGateRenorm)) {
#define MOK_SMALL_G(SG, RN)                                                                                     \
  launch_small_variant<SG, RN>(s, logits, T, E, k, eb, ee, nbits, idx_out, gate_out, idx_saved, gate_saved, lse, \
                               counts_out, offsets_out, offsets_saved, tile_prefix, expert_order, row_of_pair,     \
                               pair_of_row, status)
    case 0: MOK_SMALL_G(false, false); break;
    case kGateSigmoid: MOK_SMALL_G(true, false); break;
    case kGateRenorm: MOK_SMALL_G(false, true); break;
    default: MOK_SMALL_G(true, true); break;
#undef MOK_SMALL_G
  }
  return hipGetLastError();
}

hipError_t launch_counting_sort(const int32_t* idx, int T, int k, int E, int eb, int ee, int nchunks,
                                int32_t* chunk_counts, int32_t* chunk_base, int32_t* counts_out,
                                int32_t* offsets_out, int32_t* offsets_saved, int32_t* tile_prefix,
                                int32_t* expert_order, int32_t* row_of_pair, int32_t* pair_of_row, hipStream_t s) {
  const int64_t npairs = (int64_t)T * k;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int blocks = (nchunks + 3) / 4;
  const size_t smem = (size_t)4 * E * sizeof(int32_t);
  if (blocks > 0) {
    hipLaunchKernelGGL(sort_hist_kernel, dim3(blocks), dim3(256), smem, s, idx, npairs, E, eb, ee, nbits,
                       nchunks, chunk_counts);
  }
  hipLaunchKernelGGL(sort_scan_kernel, dim3(1), dim3(1024), 0, s, chunk_counts, nchunks, E, eb, ee,
                     chunk_base, counts_out, offsets_out, offsets_saved, tile_prefix, expert_order);
  if (blocks > 0) {
    hipLaunchKernelGGL(sort_scatter_kernel, dim3(blocks), dim3(256), smem, s, idx, npairs, E, eb, ee, nbits,
                       nchunks, chunk_base, row_of_pair, pair_of_row);
  }
  return hipGetLastError();
}

}  // namespace mok
