// Weight-streaming expert GEMMs for forward calls with few rows per expert (a
// decode step).  With tens of rows per expert the two forward products are
// bound by reading the experts' weights from HBM once, not by the matrix
// cores; the tiled kernels' 256-row tiles would then spend most of their MFMA
// work on padding and leave most compute units idle.  Here a workgroup takes
// one (32-row tile of an expert, 16 * NWN weight rows) unit at a time and
// streams those weight rows once, straight from HBM into registers:
//   UP    H = silu(X W1^T) * (X W3^T)   (x rows pulled through pair_of_row;
//                                         A = X W1^T and B = X W3^T saved
//                                         when the call saves for backward)
//   DOWN  Y = H W2^T
// Both weight matrices hold K contiguous per output column (W1, W3: [F, d];
// W2: [d, F]), so a lane reads 64 contiguous bytes of one weight row per
// 128-K chunk.  Products on v_mfma_f32_16x16x32_bf16: the lane holding
// weight row n (lane % 16) and K-group g (lane / 16) feeds the MFMA B operand,
// the lane holding activation row lane % 16 of the same K-group the A
// operand; inside a 128-K chunk, K-group g's 32 elements are the MFMA K steps
// s = 0..3 (eight each), the same K permutation on both operands, so every
// product term is summed exactly once.  KS waves split the K range of one
// 16-column group; their fp32 partial sums meet in LDS and are added in wave
// order (0 + 1 + 2 + 3), so the result is run-to-run identical.
#include "gemm_common.h"
#include "gemm_pipe.h"
#include "mok_device.h"

namespace mok {
namespace {

constexpr int kChunkK = 128;  // K elements per lane-group round (64 bytes per lane)

// Chunks in flight ahead of the one being multiplied (registers: NB + RG
// 16-byte quads x 4 per chunk and lane).  One: the occupancy it leaves (three
// workgroups per CU for UP with one row group) moves more bytes than deeper
// rings at two (same-box A/B at d 4096, E 128, k 8, F 1536: UP 36.0 / 46.0 /
// 46.2 us at T 1 for depths 1 / 2 / 3, 166 / 185 / 186 us at T 8).  DOWN
// splits K over two waves at most (F / 2 per wave; splits 1 / 2 / 4: 41.1 /
// 22.2 / 23.6 us at T 1, 260 / 256 / 272 us at T 64).  For scale: a plain
// grid-stride read of 4 GiB on the same box reaches 5.3-6.3 TB/s; UP at T 8
// moves 5.9 TB/s.
#ifndef MOK_STREAM_DEPTH
#define MOK_STREAM_DEPTH 1
#endif
#ifndef MOK_STREAM_KS_DOWN
#define MOK_STREAM_KS_DOWN 2
#endif

// RG: 16-row groups per tile that the kernel multiplies (1 when no expert can
// have more than 16 rows, T <= 16; else 2, the whole 32-row tile).
template <int KIND, int KS, int RG>
__global__ __launch_bounds__(256) void stream_gemm_kernel(GroupedGemmArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NB = Traits<KIND>::NB;  // UP pairs W1 with W3
  constexpr int NWN = 4 / KS;           // 16-column groups per workgroup
  constexpr int D = MOK_STREAM_DEPTH, NBUF = D + 1;
  const GemmGeom G = geom_of<KIND>(a.d, a.F);
  const int N = G.N, K = G.K;
  const int ntn = N / (16 * NWN);
  const int E_loc = a.E_loc;
  const int32_t* tp = a.tile_prefix + kStreamTileTable * (E_loc + 1);
  const int total = sload(tp + E_loc) * ntn;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int cg = w % NWN, kr = w / NWN;
  const int kw = K / KS;  // this wave's K range: [kr * kw, (kr + 1) * kw)
  const int nchunk = kw / kChunkK;
  const int r16 = lane & 15, g4 = lane >> 4;
  __shared__ f32x4_t red[KS > 1 ? (KS - 1) * NWN : 1][RG][NB][64];

  // XCD-aware order: workgroup b (on XCD b % 8) takes the units of the
  // contiguous run [x G/8, (x+1) G/8) of each round of G units, so that the
  // row tiles of one expert and weight rows (adjacent units) share one L2.
  const int Gd = gridDim.x;
  const int vb = (Gd % 8 == 0) ? (blockIdx.x % 8) * (Gd / 8) + blockIdx.x / 8 : blockIdx.x;
  for (int u = vb; u < total; u += Gd) {
    // expert: the last local expert whose first unit is at or before u (its
    // units [tp[e] ntn, tp[e+1] ntn), column group major, row tile minor)
    const int q = u / ntn;
    int lo = 0, hi = E_loc - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sload(tp + mid) <= q) lo = mid; else hi = mid - 1;
    }
    const int t0 = sload(tp + lo), nte = sload(tp + lo + 1) - t0;
    const int li = u - t0 * ntn;
    const int mt = li % nte, nt = li / nte;
    const int e = a.eb + lo;
    const int row0 = sload(a.offsets + e) + mt * kStreamTileRows;
    const int erow_end = sload(a.offsets + e + 1);
    const int row_end = erow_end < row0 + 16 * RG ? erow_end : row0 + 16 * RG;
    const bool two = RG == 2 && row_end - row0 > 16;  // the tile's second 16-row group is used
    const int n0 = (nt * NWN + cg) * 16;

    // operand rows of this lane, at its first K element
    const int64_t kb = (int64_t)kr * kw + 32 * g4;
    const bf16_t* bp[NB];
    bp[0] = (const bf16_t*)a.B0 + (int64_t)lo * G.b_estride + (int64_t)(n0 + r16) * G.ldb + kb;
    if constexpr (NB == 2) bp[1] = (const bf16_t*)a.B1 + (int64_t)lo * G.b_estride + (int64_t)(n0 + r16) * G.ldb + kb;
    const bf16_t* ap[RG];
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
      int r = row0 + 16 * gi + r16;
      if (r >= row_end) r = row0;  // padding rows repeat the first row; never stored
      int64_t src = r;
      if constexpr (KIND == KIND_UP) src = a.gather_rows[r] / a.k_top;  // pull dispatch: the token's x row
      ap[gi] = (const bf16_t*)a.A + src * G.lda + kb;
    }

    f32x4_t acc[RG][NB];
#pragma unroll
    for (int gi = 0; gi < RG; ++gi)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[gi][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t bq[NBUF][NB][4], aq[NBUF][RG][4];
    auto load = [&](int buf, int c) {
      const int64_t ko = (int64_t)c * kChunkK;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) bq[buf][b][j] = *reinterpret_cast<const u32x4_t*>(bp[b] + ko + 8 * j);
#pragma unroll
      for (int j = 0; j < 4; ++j) aq[buf][0][j] = *reinterpret_cast<const u32x4_t*>(ap[0] + ko + 8 * j);
      if constexpr (RG == 2)
        if (two)
#pragma unroll
          for (int j = 0; j < 4; ++j) aq[buf][RG - 1][j] = *reinterpret_cast<const u32x4_t*>(ap[RG - 1] + ko + 8 * j);
    };
    auto compute = [&](int buf) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const bf16x8_t bf = __builtin_bit_cast(bf16x8_t, bq[buf][b][s]);
          acc[0][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, aq[buf][0][s]), bf,
                                                              acc[0][b], 0, 0, 0);
          if constexpr (RG == 2)
            if (two)
              acc[RG - 1][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, aq[buf][RG - 1][s]), bf, acc[RG - 1][b], 0, 0, 0);
        }
    };
    // a ring of NBUF register buffers: chunk c + D is in flight while c is used
#pragma unroll
    for (int i = 0; i < D; ++i)
      if (i < nchunk) load(i, i);
    for (int c = 0; c < nchunk; c += NBUF) {
#pragma unroll
      for (int bb = 0; bb < NBUF; ++bb) {
        if (c + bb < nchunk) {
          if (c + bb + D < nchunk) load((bb + D) % NBUF, c + bb + D);
          compute(bb);
        }
      }
    }

    if constexpr (KS > 1) {
      if (kr > 0)
#pragma unroll
        for (int gi = 0; gi < RG; ++gi)
#pragma unroll
          for (int b = 0; b < NB; ++b) red[(kr - 1) * NWN + cg][gi][b][lane] = acc[gi][b];
      __syncthreads();
      if (kr == 0)
#pragma unroll
        for (int qk = 1; qk < KS; ++qk)
#pragma unroll
          for (int gi = 0; gi < RG; ++gi)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[gi][b] += red[(qk - 1) * NWN + cg][gi][b][lane];
      __syncthreads();  // the partials are read before the next unit writes them
    }
    if (kr == 0) {
      // D layout of the 16x16 MFMA: lane holds column lane % 16, rows 4 (lane / 16) + i
      const int col = n0 + r16;
#pragma unroll
      for (int gi = 0; gi < RG; ++gi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = row0 + 16 * gi + 4 * g4 + i;
          if (row < row_end) {
            const int64_t o = (int64_t)row * N + col;
            if constexpr (KIND == KIND_UP) {
              const float va = acc[gi][0][i], vb_ = acc[gi][1][i];
              ((bf16_t*)a.out0)[o] = f2bf(va * sigmoidf_(va) * vb_);
              if (a.save) {
                ((bf16_t*)a.save_a)[o] = f2bf(va);
                ((bf16_t*)a.save_b)[o] = f2bf(vb_);
              }
            } else {
              ((bf16_t*)a.out0)[o] = f2bf(acc[gi][0][i]);
            }
          }
        }
    }
  }
#endif
}

template <int KIND, int KS, int RG>
hipError_t run_stream(const GroupedGemmArgs& g, hipStream_t s) {
  constexpr int NWN = 4 / KS;
  const GemmGeom G = geom_of<KIND>(g.d, g.F);
  const int64_t ntn = G.N / (16 * NWN);
  const int64_t worst = ((g.P_max + kStreamTileRows - 1) / kStreamTileRows + g.E_loc) * ntn;
  // persistent workgroups: as many as fit on the device at once
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stream_gemm_kernel<KIND, KS, RG>, 256, 0) != hipSuccess ||
        n < 1)
      n = 1;
    return n;
  }();
  const int64_t cap = (int64_t)kNumCUs * per_cu;
  const int blocks = (int)(worst < cap ? worst : cap);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((stream_gemm_kernel<KIND, KS, RG>), dim3(blocks), dim3(256), 0, s, g);
  return hipGetLastError();
}

template <int KIND, int RG>
hipError_t run_stream_k(int ks, const GroupedGemmArgs& g, hipStream_t s) {
  switch (ks) {
    case 4: return run_stream<KIND, 4, RG>(g, s);
    case 2: return run_stream<KIND, 2, RG>(g, s);
    case 1: return run_stream<KIND, 1, RG>(g, s);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ MXFP8 / MXFP4
// The same weight streaming for MX weights (E4M3 codes, or E2M1 codes two
// per byte, with one E8M0 scale per 32 along K, pair-plane scales as
// mok_quantize_mxfp8 / mok_quantize_mxfp4 write them), on
// v_mfma_scale_f32_32x32x64_f8f6f4: a unit is (32-row tile, 32 * NWN weight
// rows) and K steps of 64 values.  The instruction's operand layout (as the
// tiled MX GEMMs feed it): lane l holds row l % 32 and, with h = l / 32,
// E4M3: bytes [16 h, 16 h + 16) and [32 + 16 h, 48 + 16 h) of the step;
// E2M1: bytes [16 h, 16 h + 16) of the step's 32; and the scale of the
// step's 32-block h.  Loads go in chunks of CS steps, 128 bytes of each
// operand row (64 per lane), the next chunk in flight while one is
// multiplied.  UP quantises H along F in its epilogue (one 32-column block
// per column group: the unit's rows of H are whole MX blocks) for DOWN,
// which writes bf16 Y.  Forward only (no saved A, B, H).
template <int KIND, int KS, int FMT, int D>
__global__ __launch_bounds__(256) void stream_mx_kernel(GroupedGemmArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NB = Traits<KIND>::NB;
  constexpr int NWN = 4 / KS;  // 32-column groups per workgroup
  constexpr bool FP4 = FMT == 4;
  constexpr int EPB = FP4 ? 2 : 1;  // K values per byte
  constexpr int SB = 64 / EPB;      // bytes of one MFMA K step
  constexpr int CS = 2 * EPB;       // steps per chunk: 128 bytes of a row
  const int N = KIND == KIND_UP ? a.F : a.d, K = KIND == KIND_UP ? a.d : a.F;
  const int Kb = K / EPB;  // bytes per operand row
  const int ntn = N / (32 * NWN);
  const int E_loc = a.E_loc;
  const int32_t* tp = a.tile_prefix + kStreamTileTable * (E_loc + 1);
  const int total = sload(tp + E_loc) * ntn;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int cg = w % NWN, kr = w / NWN;
  const int kw = Kb / KS;       // bytes of K per wave
  const int nstep = kw / SB;    // MFMA K steps per wave
  const int nch = (nstep + CS - 1) / CS;
  const int r32 = lane & 31, h = lane >> 5;
  __shared__ f32x16_t red[KS > 1 ? (KS - 1) * NWN : 1][NB][64];
  __shared__ float hs[NWN][32][33];  // UP: H of a column group, 32 rows x 32 columns (+1: no bank conflicts)
  const int64_t a_planes = a.P_max * 2;                        // bytes per scale plane of A (P_max rows)
  const int64_t b_planes = (int64_t)E_loc * N * 2;             // of the weights
  const int Gd = gridDim.x;
  const int vb = (Gd % 8 == 0) ? (blockIdx.x % 8) * (Gd / 8) + blockIdx.x / 8 : blockIdx.x;
  for (int u = vb; u < total; u += Gd) {
    const int q = u / ntn;
    int lo = 0, hi = E_loc - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sload(tp + mid) <= q) lo = mid; else hi = mid - 1;
    }
    const int t0 = sload(tp + lo), nte = sload(tp + lo + 1) - t0;
    const int li = u - t0 * ntn;
    const int mt = li % nte, nt = li / nte;
    const int e = a.eb + lo;
    const int row0 = sload(a.offsets + e) + mt * kStreamTileRows;
    const int erow_end = sload(a.offsets + e + 1);
    const int row_end = erow_end < row0 + 32 ? erow_end : row0 + 32;
    const int n0 = (nt * NWN + cg) * 32;
    // this lane's operand rows: A row (padding rows repeat the first; never
    // stored) and weight row n0 + r32, at the wave's first K byte
    const int arow = row0 + r32 < row_end ? row0 + r32 : row0;
    const int64_t kb = (int64_t)kr * kw;
    const uint8_t* ap = (const uint8_t*)a.A + (int64_t)arow * Kb + kb;
    const int64_t wrow = (int64_t)lo * N + n0 + r32;
    const uint8_t* bp0 = (const uint8_t*)a.B0 + wrow * Kb + kb;
    const uint8_t* bp1 = NB == 2 ? (const uint8_t*)a.B1 + wrow * Kb + kb : bp0;
    const uint8_t* asc = a.a_scale + (int64_t)arow * 2 + h;
    const uint8_t* bsc0 = a.b_scale0 + wrow * 2 + h;
    const uint8_t* bsc1 = NB == 2 ? a.b_scale1 + wrow * 2 + h : bsc0;
    const int p0 = kr * nstep;  // the wave's first scale plane

    f32x16_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][i] = 0.f;
    // per step and operand: E4M3 the lane's two 16-byte pieces, E2M1 its one
    // (the operand's upper half is not read for E2M1 and stays zero)
    constexpr int NQ = FP4 ? 1 : 2;
    constexpr int NBUF = D + 1;  // chunk c + D is in flight while c is multiplied
    i32x4_t av[NBUF][CS][NQ], bv[NBUF][CS][NB][NQ];
    int as_[NBUF][CS], bs_[NBUF][CS][NB];
    auto ld = [&](i32x4_t (&dst)[NQ], const uint8_t* p, int st) {
      const int64_t o = (int64_t)st * SB + 16 * h;
#pragma unroll
      for (int qq = 0; qq < NQ; ++qq) dst[qq] = *reinterpret_cast<const i32x4_t*>(p + o + 32 * qq);
    };
    auto op = [&](const i32x4_t (&v)[NQ]) -> i32x8_t {
      if constexpr (FP4) {
        const i32x4_t z = {0, 0, 0, 0};
        return __builtin_shufflevector(v[0], z, 0, 1, 2, 3, 4, 5, 6, 7);
      } else {
        return __builtin_shufflevector(v[0], v[NQ - 1], 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
    auto load = [&](int buf, int c) {
#pragma unroll
      for (int j = 0; j < CS; ++j) {
        const int st = c * CS + j;
        if (st < nstep) {
          ld(av[buf][j], ap, st);
          as_[buf][j] = asc[(int64_t)(p0 + st) * a_planes];
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            ld(bv[buf][j][b], b ? bp1 : bp0, st);
            bs_[buf][j][b] = (b ? bsc1 : bsc0)[(int64_t)(p0 + st) * b_planes];
          }
        }
      }
    };
    auto compute = [&](int buf, int c) {
#pragma unroll
      for (int j = 0; j < CS; ++j)
        if (c * CS + j < nstep)
#pragma unroll
          for (int b = 0; b < NB; ++b)
            acc[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op(av[buf][j]), op(bv[buf][j][b]), acc[b], FMT,
                                                                      FMT, 0, as_[buf][j], 0, bs_[buf][j][b]);
    };
#pragma unroll
    for (int i = 0; i < D; ++i)
      if (i < nch) load(i, i);
    for (int c = 0; c < nch; c += NBUF) {
#pragma unroll
      for (int bb = 0; bb < NBUF; ++bb) {
        if (c + bb < nch) {
          if (c + bb + D < nch) load((bb + D) % NBUF, c + bb + D);
          compute(bb, c + bb);
        }
      }
    }

    if constexpr (KS > 1) {
      if (kr > 0)
#pragma unroll
        for (int b = 0; b < NB; ++b) red[(kr - 1) * NWN + cg][b][lane] = acc[b];
      __syncthreads();
      if (kr == 0)
#pragma unroll
        for (int qk = 1; qk < KS; ++qk)
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[b] += red[(qk - 1) * NWN + cg][b][lane];
      __syncthreads();  // the partials are read before the next unit writes them
    }
    if (kr == 0) {
      // lane holds column n0 + r32 of rows (i / 4) 8 + 4 h + i % 4
      if constexpr (KIND == KIND_UP) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float va = acc[0][i], vb_ = acc[1][i];
          hs[cg][(i >> 2) * 8 + 4 * h + (i & 3)][r32] = va * sigmoidf_(va) * vb_;
        }
        __builtin_amdgcn_wave_barrier();
        if (lane < 32 && row0 + lane < row_end) {
          // lane r quantises row r of the block: 32 values, one MX block
          float v[32];
          float amax = 0.f;
#pragma unroll
          for (int c = 0; c < 32; ++c) {
            v[c] = hs[cg][lane][c];
            amax = fmaxf(amax, fabsf(v[c]));
          }
          const int row = row0 + lane;
          int se;
          if constexpr (FP4) {
            se = mx4_scale_exp(amax);
            u32x4_t wq;
#pragma unroll
            for (int j = 0; j < 4; ++j) wq[j] = e2m1x8(v + 8 * j, se);
            *reinterpret_cast<u32x4_t*>((uint8_t*)a.out0 + (int64_t)row * (N / 2) + n0 / 2) = wq;
          } else {
            se = mx_scale_exp(amax);
            uint8_t* dst = (uint8_t*)a.out0 + (int64_t)row * N + n0;
#pragma unroll
            for (int q4 = 0; q4 < 2; ++q4) {
              u32x4_t wq;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int c = 16 * q4 + 4 * j;
                wq[j] = e4m3x4(ldexpf(v[c], -se), ldexpf(v[c + 1], -se), ldexpf(v[c + 2], -se), ldexpf(v[c + 3], -se));
              }
              *reinterpret_cast<u32x4_t*>(dst + 16 * q4) = wq;
            }
          }
          const int blk = n0 / 32;  // H scales: pair planes [F / 64, P_max, 2]
          a.out_scale[(int64_t)(blk >> 1) * a.P_max * 2 + (int64_t)row * 2 + (blk & 1)] = (uint8_t)(se + 127);
        }
        __builtin_amdgcn_wave_barrier();
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = row0 + (i >> 2) * 8 + 4 * h + (i & 3);
          if (row < row_end) ((bf16_t*)a.out0)[(int64_t)row * N + n0 + r32] = f2bf(acc[0][i]);
        }
      }
    }
  }
#endif
}

template <int KIND, int KS, int FMT, int D>
hipError_t run_stream_mx(const GroupedGemmArgs& g, hipStream_t s) {
  constexpr int NWN = 4 / KS;
  const int N = KIND == KIND_UP ? g.F : g.d;
  const int64_t ntn = N / (32 * NWN);
  const int64_t worst = ((g.P_max + kStreamTileRows - 1) / kStreamTileRows + g.E_loc) * ntn;
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stream_mx_kernel<KIND, KS, FMT, D>, 256, 0) != hipSuccess ||
        n < 1)
      n = 1;
    return n;
  }();
  const int64_t cap = (int64_t)kNumCUs * per_cu;
  const int blocks = (int)(worst < cap ? worst : cap);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((stream_mx_kernel<KIND, KS, FMT, D>), dim3(blocks), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

int stream_ksplit(int K) {
  if (K % (kChunkK * 4) == 0) return 4;
  if (K % (kChunkK * 2) == 0) return 2;
  if (K % kChunkK == 0) return 1;
  return 0;
}

// MX weight streaming: waves splitting K (UP, DOWN) and chunks in flight,
// per operand format.
#ifndef MOK_MX8_STREAM_KS_UP
#define MOK_MX8_STREAM_KS_UP 4
#endif
#ifndef MOK_MX8_STREAM_KS_DOWN
#define MOK_MX8_STREAM_KS_DOWN 2
#endif
#ifndef MOK_MX8_STREAM_DEPTH
#define MOK_MX8_STREAM_DEPTH 1
#endif
#ifndef MOK_MX4_STREAM_KS_UP
#define MOK_MX4_STREAM_KS_UP 4
#endif
#ifndef MOK_MX4_STREAM_KS_DOWN
#define MOK_MX4_STREAM_KS_DOWN 2
#endif
#ifndef MOK_MX4_STREAM_DEPTH
#define MOK_MX4_STREAM_DEPTH 1
#endif
constexpr int kMaxKsUp = MOK_MX8_STREAM_KS_UP > MOK_MX4_STREAM_KS_UP ? MOK_MX8_STREAM_KS_UP : MOK_MX4_STREAM_KS_UP;
constexpr int kMaxKsDown =
    MOK_MX8_STREAM_KS_DOWN > MOK_MX4_STREAM_KS_DOWN ? MOK_MX8_STREAM_KS_DOWN : MOK_MX4_STREAM_KS_DOWN;

// Each wave's K range is a whole number of 64-value steps (E4M3 64 bytes,
// E2M1 32): d a multiple of 64 times UP's split, F of 64 times DOWN's.
int stream_mx_ok(int d, int F) { return d % (64 * kMaxKsUp) == 0 && F % (64 * kMaxKsDown) == 0; }

hipError_t gemm_stream_mxfp8(int kind, const GroupedGemmArgs& g, hipStream_t s) {
  if (kind == KIND_UP) return run_stream_mx<KIND_UP, MOK_MX8_STREAM_KS_UP, 0, MOK_MX8_STREAM_DEPTH>(g, s);
  if (kind == KIND_DOWN) return run_stream_mx<KIND_DOWN, MOK_MX8_STREAM_KS_DOWN, 0, MOK_MX8_STREAM_DEPTH>(g, s);
  return hipErrorInvalidValue;
}

hipError_t gemm_stream_mxfp4(int kind, const GroupedGemmArgs& g, hipStream_t s) {
  if (kind == KIND_UP) return run_stream_mx<KIND_UP, MOK_MX4_STREAM_KS_UP, 4, MOK_MX4_STREAM_DEPTH>(g, s);
  if (kind == KIND_DOWN) return run_stream_mx<KIND_DOWN, MOK_MX4_STREAM_KS_DOWN, 4, MOK_MX4_STREAM_DEPTH>(g, s);
  return hipErrorInvalidValue;
}

hipError_t gemm_stream_bf16(int kind, const GroupedGemmArgs& g, hipStream_t s) {
  // an expert holds at most one row per token: with T <= 16 every tile has
  // at most 16 rows
  const bool one_group = g.P_max / (g.k_top > 0 ? g.k_top : 1) <= 16;
  if (kind == KIND_UP) {
    const int ks = stream_ksplit(g.d);
    return one_group ? run_stream_k<KIND_UP, 1>(ks, g, s) : run_stream_k<KIND_UP, 2>(ks, g, s);
  }
  if (kind == KIND_DOWN) {
    int ks = stream_ksplit(g.F);
    if (ks > MOK_STREAM_KS_DOWN) ks = MOK_STREAM_KS_DOWN;
    return one_group ? run_stream_k<KIND_DOWN, 1>(ks, g, s) : run_stream_k<KIND_DOWN, 2>(ks, g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mok
