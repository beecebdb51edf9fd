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
// Tiling: a workgroup of 4 waves (2 x 2) computes a BM x BN tile (per B
// matrix; UP computes the W1 and W3 tiles of the same columns), each wave a
// (BM/2) x (BN/2) block of 32x32 MFMA tiles, over K in steps of 64 staged
// through double-buffered LDS in a K-contiguous [row][k] layout: 128-byte rows
// of eight 16-byte chunks, XOR-swizzled so that the 16-byte fragment reads of
// 16 consecutive rows hit distinct banks.  Operands stored K-contiguous go
// from HBM straight to LDS (buffer_load_dwordx4 ... lds, 1 KB per wave
// instruction, no VGPRs), through buffer resources rebased on each tile so
// that rows past the expert's end read as zero.  Operands stored M- or
// N-contiguous (the backward products) are loaded as 8 x 8 blocks and
// transposed in registers (v_perm_b32) before 16-byte LDS stores.
//
// Scheduling: row-grouped kinds run a persistent loop over the tiles of all
// local experts in (expert, n-tile, m-tile) order, with the tile prefix of
// each expert computed on the device by the counting sort, so the host never
// needs the data-dependent row count.  Workgroup b runs on XCD b mod 8; the
// loop hands each XCD a contiguous run of tiles so that m-tiles sharing a
// weight tile meet in one L2.  Every output element is produced by one
// workgroup with a fixed K order: results are run-to-run identical (no
// split-K, no atomics).
#include "mok_device.h"
#include "mok_internal.h"
#include "gemm_common.h"

namespace mok {

constexpr int kBK = 64;           // K step; one LDS row holds 64 bf16 = 128 bytes = 8 chunks
constexpr int kRowBytes = kBK * 2;

// Physical 16-byte chunk of logical chunk c in LDS row r.  This XOR swizzle
// keeps fragment reads (32 consecutive rows, one chunk) and the transposed
// block stores below free of bank conflicts for 64 banks with 16-lane phases
// and for 32 banks with 8-lane phases alike.
__device__ __forceinline__ int swz_chunk(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

// Grouped raster inside one expert: groups of GM m-tiles, n-tiles outer and
// m-tiles inner within a group, so that a run of consecutive tiles forms a
// GM x (run / GM) block that reuses both operands.
__device__ __forceinline__ void tile_mn(int local, int mt, int ntn, int& m, int& n) {
  constexpr int GM = 4;
  const int g = local / (GM * ntn);
  const int gm0 = g * GM;
  const int gsz = mt - gm0 < GM ? mt - gm0 : GM;
  const int rem = local - g * GM * ntn;
  n = rem / gsz;
  m = gm0 + rem % gsz;
}

// Store the transpose of an 8 x 8 block of 16-bit values into a swizzled LDS
// tile: in[i] holds K-row i (8 consecutive M/N values starting at 8 * mb);
// LDS row 8 * mb + t receives chunk kb = those 8 K values of column t.
// Lanes with bit 3 of mb set write the rows of each pair in swapped order,
// which removes the remaining bank conflicts (only the v_perm selector
// changes per lane).
__device__ __forceinline__ void transposed_store(const u32x4_t in[8], uint8_t* tile, int mb, int kb) {
  const uint32_t x = (mb >> 3) & 1;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int t = j ^ (int)x;
    const uint32_t sel = ((j & 1) ^ x) ? 0x07060302u : 0x05040100u;
    u32x4_t o;
#pragma unroll
    for (int w = 0; w < 4; ++w) o[w] = __builtin_amdgcn_perm(in[2 * w + 1][j >> 1], in[2 * w][j >> 1], sel);
    const int r = mb * 8 + t;
    *reinterpret_cast<u32x4_t*>(&tile[r * kRowBytes + swz_chunk(r, kb) * 16]) = o;
  }
}

template <int KIND, int BM, int BN>
struct TileCfg {
  using Tr = Traits<KIND>;
  static constexpr int NT = 256, WM = 2, WN = 2;
  static constexpr int NB = Tr::NB;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int BROWS = NB * BN;
  // K-contiguous operand: direct-to-LDS loads of 8 rows (1 KB) per wave instruction
  static constexpr int DMA_A = Tr::A_MN ? 0 : BM / 8 / 4;
  static constexpr int DMA_B = Tr::B_MN ? 0 : BROWS / 8 / 4;
  // MN-contiguous operand: 8x8 blocks per thread, transposed in registers
  static constexpr int BLA = Tr::A_MN ? (kBK / 8) * (BM / 8) / NT : 0;
  static constexpr int BLB = Tr::B_MN ? (kBK / 8) * (BROWS / 8) / NT : 0;
  static_assert(!Tr::A_MN || BLA >= 1, "MN tile too small");
  static_assert(!Tr::B_MN || BLB >= 1, "MN tile too small");
  static_assert(BM % 32 == 0 && BROWS % 32 == 0, "tile rows");
};

// One output tile: K loop over double-buffered LDS stages, then the
// LDS-staged epilogue.  Called by every thread of the workgroup with
// wave-uniform tile coordinates; ends with a barrier (the epilogue staging
// overlaps the next tile's first K stage).
template <int KIND, int BM, int BN>
__device__ __forceinline__ void gemm_tile(const GroupedGemmArgs& args, uint8_t* arena, int e_loc, int row0,
                                          int row_end, int m0, int n0, int z) {
  using Tr = Traits<KIND>;
  using C = TileCfg<KIND, BM, BN>;
  constexpr int NT = C::NT, NB = C::NB, TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN, BROWS = C::BROWS;
  uint8_t (*sA)[BM * kRowBytes] = reinterpret_cast<uint8_t (*)[BM * kRowBytes]>(arena);
  uint8_t (*sB)[BROWS * kRowBytes] = reinterpret_cast<uint8_t (*)[BROWS * kRowBytes]>(arena + 2 * BM * kRowBytes);
  const GemmGeom G = geom_of<KIND>(args.d, args.F);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps DMA operands scalar
  const int wm = wid / C::WN, wn = wid % C::WN;
  const bf16_t* __restrict__ Abase = (const bf16_t*)args.A;
  const bf16_t* __restrict__ B0 = (const bf16_t*)args.B0;
  const bf16_t* __restrict__ B1 = (const bf16_t*)args.B1;
  const int kbeg = Tr::GROUP_K ? row0 : 0;
  const int kend = Tr::GROUP_K ? row_end : G.K;
  const int nk = (kend - kbeg + kBK - 1) / kBK;

  // ------------------------------------------------------------ direct-to-LDS sources
  // Buffer resources rebased on this tile: rows past the expert's end (A) or
  // past N (B) fall outside num_records and read as zero.
  i32x4_t rsA = make_rsrc(Abase, 0u);
  i32x4_t rsB0 = rsA, rsB1 = rsA;
  uint32_t offA[C::DMA_A > 0 ? C::DMA_A : 1], offB[C::DMA_B > 0 ? C::DMA_B : 1];
  if constexpr (!Tr::A_MN) {
    const int rows = row_end - row0 < BM ? row_end - row0 : BM;  // this tile's rows
    if (args.gather_rows) {
      // pull dispatch: each row comes straight from its token's row of x
      rsA = make_rsrc(Abase, (uint32_t)(args.gather_src_rows * G.lda * 2));
#pragma unroll
      for (int q = 0; q < C::DMA_A; ++q) {
        const int r = (wid * C::DMA_A + q) * 8 + (lane >> 3);
        const int tok = r < rows ? args.gather_rows[row0 + r] / args.k_top : -1;
        offA[q] = tok >= 0 ? (uint32_t)(tok * G.lda * 2 + swz_chunk(r, lane & 7) * 16) : 0xFFFFFFF0u;
      }
    } else {
      rsA = make_rsrc(Abase + ((int64_t)row0 - args.a_row_shift) * G.lda, (uint32_t)((int64_t)rows * G.lda * 2));
#pragma unroll
      for (int q = 0; q < C::DMA_A; ++q) {
        const int r = (wid * C::DMA_A + q) * 8 + (lane >> 3);
        offA[q] = (uint32_t)(r * G.lda * 2 + swz_chunk(r, lane & 7) * 16);
      }
    }
  }
  if constexpr (!Tr::B_MN) {
    const int nb_rows = G.N - n0 < BN ? G.N - n0 : BN;  // this tile's rows of each B matrix
    const bf16_t* b0 = B0 + (int64_t)e_loc * G.b_estride + (int64_t)n0 * G.ldb;
    rsB0 = make_rsrc(b0, (uint32_t)((int64_t)nb_rows * G.ldb * 2));
    if constexpr (NB == 2) {
      const bf16_t* b1 = B1 + (int64_t)e_loc * G.b_estride + (int64_t)n0 * G.ldb;
      rsB1 = make_rsrc(b1, (uint32_t)((int64_t)nb_rows * G.ldb * 2));
    }
#pragma unroll
    for (int q = 0; q < C::DMA_B; ++q) {
      const int r = (wid * C::DMA_B + q) * 8 + (lane >> 3);      // LDS row
      const int rl = (NB == 2 && r >= BN) ? r - BN : r;          // row within its matrix
      offB[q] = (uint32_t)(rl * G.ldb * 2 + swz_chunk(r, lane & 7) * 16);
    }
  }

  u32x4_t ta[C::BLA > 0 ? C::BLA : 1][8], tb[C::BLB > 0 ? C::BLB : 1][8];

  // Issue the loads of K-step k0 into LDS stage `buf` (direct) or registers (MN).
  auto issue = [&](int k0, int buf) {
    if constexpr (!Tr::A_MN) {
#pragma unroll
      for (int q = 0; q < C::DMA_A; ++q)
        dma_b128(rsA, lds_addr(&sA[buf][(wid * C::DMA_A + q) * 1024]), offA[q], k0 * 2);
    } else {
      const bf16_t* p = Abase + (KIND == KIND_DW13 ? (int64_t)z * args.F : 0);
#pragma unroll
      for (int q = 0; q < C::BLA; ++q) {
        const int blk = tid + q * NT;
        const int mb = blk % (BM / 8), kb = blk / (BM / 8);
        const int m = m0 + mb * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int kr = k0 + kb * 8 + i;
          ta[q][i] = (kr < kend && m < G.M) ? *reinterpret_cast<const u32x4_t*>(p + (int64_t)kr * G.lda + m)
                                            : u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
    if constexpr (!Tr::B_MN) {
#pragma unroll
      for (int q = 0; q < C::DMA_B; ++q) {
        const int r = (wid * C::DMA_B + q) * 8;
        dma_b128((NB == 2 && r >= BN) ? rsB1 : rsB0, lds_addr(&sB[buf][(wid * C::DMA_B + q) * 1024]), offB[q],
                 k0 * 2);
      }
    } else {
#pragma unroll
      for (int q = 0; q < C::BLB; ++q) {
        const int blk = tid + q * NT;
        const int nb = blk % (BROWS / 8), kb = blk / (BROWS / 8);
        const int n = n0 + nb * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int kr = k0 + kb * 8 + i;
          const bf16_t* src;
          bool ok;
          if constexpr (!Tr::GROUP_K) {
            const int krl = kr < G.ksplit ? kr : kr - G.ksplit;
            src = (kr < G.ksplit ? B0 : B1) + (int64_t)e_loc * G.b_estride + (int64_t)krl * G.ldb + n;
            ok = n < G.N;
          } else {
            ok = kr < kend && n < G.N;
            // ring mode keeps no expert-sorted copy of X: pull the token rows
            const int64_t srow = args.gather_rows ? (ok ? args.gather_rows[kr] / args.k_top : 0) : kr;
            src = B0 + srow * G.ldb + n;
          }
          tb[q][i] = ok ? *reinterpret_cast<const u32x4_t*>(src) : u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  // Transpose the register-staged (MN) blocks into LDS stage `buf`.
  auto commit = [&](int buf) {
    if constexpr (Tr::A_MN) {
#pragma unroll
      for (int q = 0; q < C::BLA; ++q) {
        const int blk = tid + q * NT;
        transposed_store(ta[q], sA[buf], blk % (BM / 8), blk / (BM / 8));
      }
    }
    if constexpr (Tr::B_MN) {
#pragma unroll
      for (int q = 0; q < C::BLB; ++q) {
        const int blk = tid + q * NT;
        transposed_store(tb[q], sB[buf], blk % (BROWS / 8), blk / (BROWS / 8));
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
    issue(kbeg, 0);
    commit(0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) issue(kbeg + (kt + 1) * kBK, buf ^ 1);
    const uint8_t* a_s = sA[buf];
    const uint8_t* b_s = sB[buf];
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int lc = kk * 2 + (lane >> 5);
      bf16x8_t af[FM], bfr[NB][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * TM + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8_t*>(&a_s[r * kRowBytes + swz_chunk(r, lc) * 16]);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = b * BN + wn * TN + j * 32 + (lane & 31);
          bfr[b][j] = *reinterpret_cast<const bf16x8_t*>(&b_s[r * kRowBytes + swz_chunk(r, lc) * 16]);
        }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[b][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[b][j], acc[b][i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) commit(buf ^ 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // Each wave stages its accumulators in its own 32 KB LDS region, then
  // every lane handles 8 consecutive columns of one row: 16-byte loads and
  // stores along rows.
  float* ep = reinterpret_cast<float*>(arena + wid * 32768);
  const int wrow0 = wm * TM, wcol0 = wn * TN;
  if constexpr (NB == 2) {
    // UP: gate (W1) and up (W3) accumulators of one 32-column fragment
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          ep[rr * 32 + (lane & 31)] = acc[0][i][j][r];
          ep[4096 + rr * 32 + (lane & 31)] = acc[NB - 1][i][j][r];
        }
      __builtin_amdgcn_wave_barrier();
#pragma unroll 2
      for (int q = 0; q < TM * 32 / 8 / 64; ++q) {
        const int seg = q * 64 + lane;
        const int rr = seg >> 2, c8 = (seg & 3) * 8;
        const int row = row0 + wrow0 + rr, col = n0 + wcol0 + j * 32 + c8;
        if (row < row_end && col < G.N) {
          const f32x4_t* pv = reinterpret_cast<const f32x4_t*>(&ep[rr * 32 + c8]);
          const f32x4_t* pu = reinterpret_cast<const f32x4_t*>(&ep[4096 + rr * 32 + c8]);
          const f32x4_t v0 = pv[0], v1 = pv[1], u0 = pu[0], u1 = pu[1];
          float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          float u[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
          u32x4_t h, a, b;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float h0 = v[2 * t] * sigmoidf_(v[2 * t]) * u[2 * t];
            const float h1 = v[2 * t + 1] * sigmoidf_(v[2 * t + 1]) * u[2 * t + 1];
            h[t] = (uint32_t)f2bf(h0) | ((uint32_t)f2bf(h1) << 16);
            a[t] = (uint32_t)f2bf(v[2 * t]) | ((uint32_t)f2bf(v[2 * t + 1]) << 16);
            b[t] = (uint32_t)f2bf(u[2 * t]) | ((uint32_t)f2bf(u[2 * t + 1]) << 16);
          }
          const int64_t o = (int64_t)row * G.N + col;
          *reinterpret_cast<u32x4_t*>((bf16_t*)args.out0 + o) = h;
          if (args.save) {
            *reinterpret_cast<u32x4_t*>((bf16_t*)args.save_a + o) = a;
            *reinterpret_cast<u32x4_t*>((bf16_t*)args.save_b + o) = b;
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  } else {
#pragma unroll
    for (int jp = 0; jp < FN / 2; ++jp) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rr = i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            ep[rr * 64 + jj * 32 + (lane & 31)] = acc[0][i][2 * jp + jj][r];
          }
      __builtin_amdgcn_wave_barrier();
#pragma unroll 2
      for (int q = 0; q < TM * 64 / 8 / 64; ++q) {
        const int seg = q * 64 + lane;
        const int rr = seg >> 3, c8 = (seg & 7) * 8;
        const f32x4_t* pv = reinterpret_cast<const f32x4_t*>(&ep[rr * 64 + c8]);
        const f32x4_t v0 = pv[0], v1 = pv[1];
        const int col = n0 + wcol0 + jp * 64 + c8;
        if constexpr (!Tr::GROUP_K) {
          const int row = row0 + wrow0 + rr;
          if (row < row_end && col < G.N) {
            float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            const int64_t o = (int64_t)row * G.N + col;
            if constexpr (KIND == KIND_DH) {
              const u32x4_t av = *reinterpret_cast<const u32x4_t*>((const bf16_t*)args.save_a + o);
              const u32x4_t bv = *reinterpret_cast<const u32x4_t*>((const bf16_t*)args.save_b + o);
              u32x4_t da, db;
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                float dav[2], dbv[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                  const float a = __uint_as_float(hh ? (av[t] & 0xFFFF0000u) : (av[t] << 16));
                  const float b = __uint_as_float(hh ? (bv[t] & 0xFFFF0000u) : (bv[t] << 16));
                  const float sg = sigmoidf_(a);
                  const float dh = v[2 * t + hh];
                  dav[hh] = dh * b * sg * (1.0f + a * (1.0f - sg));
                  dbv[hh] = dh * a * sg;
                }
                da[t] = (uint32_t)f2bf(dav[0]) | ((uint32_t)f2bf(dav[1]) << 16);
                db[t] = (uint32_t)f2bf(dbv[0]) | ((uint32_t)f2bf(dbv[1]) << 16);
              }
              bf16_t* dab = (bf16_t*)args.out0 + (int64_t)row * 2 * args.F;
              *reinterpret_cast<u32x4_t*>(dab + col) = da;
              *reinterpret_cast<u32x4_t*>(dab + args.F + col) = db;
            } else {
              u32x4_t y;
#pragma unroll
              for (int t = 0; t < 4; ++t)
                y[t] = (uint32_t)f2bf(v[2 * t]) | ((uint32_t)f2bf(v[2 * t + 1]) << 16);
              *reinterpret_cast<u32x4_t*>((bf16_t*)args.out0 + o) = y;
            }
          }
        } else {
          const int m = m0 + wrow0 + rr;
          if (m < G.M && col < G.N) {
            float* outp = (float*)(KIND == KIND_DW13 && z ? args.out1 : args.out0);
            f32x4_t* dst = reinterpret_cast<f32x4_t*>(outp + (int64_t)e_loc * G.M * G.N + (int64_t)m * G.N + col);
            dst[0] = v0;
            dst[1] = v1;
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();  // staging regions overlap the next tile's first K stage
}

template <int KIND, int BM, int BN>
__global__ __launch_bounds__(256) void grouped_gemm_bf16_kernel(GroupedGemmArgs args) {
#if defined(__HIP_DEVICE_COMPILE__)  // device-only builtins; the host pass needs only the launch stub
  using Tr = Traits<KIND>;
  using C = TileCfg<KIND, BM, BN>;
  constexpr int NT = C::NT;

  // One LDS arena: two stages of the A and B tiles during the K loop, then
  // four per-wave staging regions for the epilogue.
  constexpr int kArena = 2 * (BM + C::BROWS) * kRowBytes;
  static_assert(kArena >= 4 * 32768, "epilogue staging needs 32 KB per wave");
  __shared__ __attribute__((aligned(1024))) uint8_t arena[kArena];
  __shared__ int32_t s_tp[1025];

  const GemmGeom G = geom_of<KIND>(args.d, args.F);
  const int tid = threadIdx.x;
  const int E_loc = args.E_loc;
  const int ntn = (G.N + BN - 1) / BN;

  int total, ntm_k = 0;
  constexpr int NZ = KIND == KIND_DW13 ? 2 : 1;  // DW13 computes dW1 (z = 0) and dW3 (z = 1)
  if constexpr (!Tr::GROUP_K) {
    const int bidx = (BM == 64) ? 0 : (BM == 128 ? 1 : 2);
    const int32_t* tp = args.tile_prefix + bidx * (E_loc + 1);
    for (int i = tid; i <= E_loc; i += NT) s_tp[i] = tp[i];
    __syncthreads();
    total = s_tp[E_loc] * ntn;
  } else {
    // this XCD's share: its experts' tiles, NZ * ntm * ntn per expert
    ntm_k = (G.M + BM - 1) / BM;
    const int x = blockIdx.x % 8;
    total = (args.expert_order[x + 1] - args.expert_order[x]) * NZ * ntm_k * ntn;
  }
  // Row-grouped kinds: equal-sized tiles in a static round-robin.  XCD-aware
  // order: workgroup b (on XCD b % 8) takes tiles from the contiguous run
  // [x * G/8, (x+1) * G/8) of each round of G tiles.  Weight-gradient kinds:
  // the work of a tile grows with its expert's rows, so the experts are dealt
  // to the XCDs longest-first (by the counting sort) and the workgroups of
  // XCD x pull that share's tiles from counter x, heaviest expert first; an
  // expert's tiles then share one L2.  Each tile is still computed whole by one
  // workgroup, so the results do not depend on the assignment.
  const int G_ = gridDim.x;
  const int vb = (G_ % 8 == 0) ? (blockIdx.x % 8) * (G_ / 8) + blockIdx.x / 8 : blockIdx.x;
  __shared__ int s_next;
  auto next_tile = [&](int cur) -> int {
    if constexpr (!Tr::GROUP_K) {
      return cur < 0 ? vb : cur + G_;
    } else {
      if (tid == 0) s_next = atomicAdd(args.queue + blockIdx.x % 8, 1);
      __syncthreads();
      const int t = s_next;
      __syncthreads();
      return t;
    }
  };

  for (int tile = next_tile(-1); tile < total; tile = next_tile(tile)) {
    int e_loc, row0, row_end, m0 = 0, n0, z = 0;
    if constexpr (!Tr::GROUP_K) {
      // (expert, n-tile, m-tile) order; expert e owns tiles [s_tp[e]*ntn, s_tp[e+1]*ntn)
      int lo = 0, hi = E_loc - 1;
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (s_tp[mid] * ntn <= tile) lo = mid; else hi = mid - 1;
      }
      e_loc = lo;
      int mt, nt;
      tile_mn(tile - s_tp[e_loc] * ntn, s_tp[e_loc + 1] - s_tp[e_loc], ntn, mt, nt);
      n0 = nt * BN;
      const int e = args.eb + e_loc;
      row0 = args.offsets[e] + mt * BM;
      row_end = args.offsets[e + 1];
    } else {
      const int per_z = ntm_k * ntn;
      e_loc = args.expert_order[16 + args.expert_order[blockIdx.x % 8] + tile / (NZ * per_z)];
      const int rem = tile % (NZ * per_z);
      z = rem / per_z;
      int mt, nt;
      tile_mn(rem % per_z, ntm_k, ntn, mt, nt);
      m0 = mt * BM;
      n0 = nt * BN;
      const int e = args.eb + e_loc;
      row0 = args.offsets[e];
      row_end = args.offsets[e + 1];
    }
    // The tile coordinates are wave-uniform; say so, so that addresses and
    // buffer resources live in scalar registers (a divergent resource would
    // make every buffer load a waterfall loop).
    e_loc = __builtin_amdgcn_readfirstlane(e_loc);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    row_end = __builtin_amdgcn_readfirstlane(row_end);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    n0 = __builtin_amdgcn_readfirstlane(n0);
    z = __builtin_amdgcn_readfirstlane(z);
    gemm_tile<KIND, BM, BN>(args, arena, e_loc, row0, row_end, m0, n0, z);
  }
#endif
}

template <int KIND, int BM, int BN>
static hipError_t run_bf16(const GroupedGemmArgs& g, hipStream_t s) {
  const GemmGeom G = geom_of<KIND>(g.d, g.F);
  const int ntn = (G.N + BN - 1) / BN;
  int blocks;
  dim3 grid;
  if constexpr (Traits<KIND>::GROUP_K) {
    // persistent workers over the 8 per-XCD tile counters (zeroed earlier on
    // the stream); a multiple of 8 workgroups so that every counter is served
    blocks = 256;
    grid = dim3(blocks);
  } else {
    // persistent: one workgroup per CU, bounded by the worst-case tile count
    const int64_t worst = ((g.P_max + BM - 1) / BM + g.E_loc) * (int64_t)ntn;
    blocks = (int)(worst < 256 ? worst : 256);
    grid = dim3(blocks);
  }
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<KIND, BM, BN>), grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t gemm_bf16(int kind, const GroupedGemmArgs& g, hipStream_t s) {
  switch (kind) {
    case KIND_UP:   return run_bf16<KIND_UP, 256, 128>(g, s);
    case KIND_DOWN: return run_bf16<KIND_DOWN, 256, 256>(g, s);
    case KIND_DH:   return run_bf16<KIND_DH, 256, 256>(g, s);
    case KIND_DX:   return run_bf16<KIND_DX, 256, 256>(g, s);
    case KIND_DW2:  return run_bf16<KIND_DW2, 256, 256>(g, s);
    case KIND_DW13: return run_bf16<KIND_DW13, 256, 256>(g, s);
  }
  return hipErrorInvalidValue;
}


// ------------------------------------------------------------------ ring pipeline
// Tile prefix of the local experts restricted to rows [r0, r1): expert i owns
// ceil(|[off_i, off_i+1) n [r0, r1)| / BM) row tiles.  256 threads, E_loc <= 1024.
template <int BM>
__device__ void range_tile_prefix(const GroupedGemmArgs& g, int r0, int r1, int32_t* s_tp, int32_t* s_wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int c[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = 4 * tid + q;
    c[q] = 0;
    if (i < g.E_loc) {
      const int lo = max(g.offsets[g.eb + i], r0), hi = min(g.offsets[g.eb + i + 1], r1);
      c[q] = hi > lo ? (hi - lo + BM - 1) / BM : 0;
    }
    sum += c[q];
  }
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) s_wsum[wid] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wid; ++w) base += s_wsum[w];
  int excl = base + incl - sum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = 4 * tid + q;
    if (i < g.E_loc) s_tp[i] = excl;
    excl += c[q];
  }
  if (tid == 255) s_tp[g.E_loc] = base + incl;
  __syncthreads();
}

// Expert and row span of tile t of a range prefix (expert-major, m fastest).
__device__ __forceinline__ void range_tile(const GroupedGemmArgs& g, const int32_t* s_tp, int ntn, int BM, int r0,
                                           int r1, int t, int& e_loc, int& row0, int& row_end, int& n0, int BN) {
  int lo = 0, hi = g.E_loc - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_tp[mid] * ntn <= t) lo = mid; else hi = mid - 1;
  }
  e_loc = lo;
  const int mt_e = s_tp[e_loc + 1] - s_tp[e_loc];
  const int local = t - s_tp[e_loc] * ntn;
  n0 = (local / mt_e) * BN;
  row0 = max(g.offsets[g.eb + e_loc], r0) + (local % mt_e) * BM;
  row_end = min(g.offsets[g.eb + e_loc + 1], r1);
}

[[maybe_unused]] constexpr int kCopyRows = 16;  // rows per mover task

__global__ __launch_bounds__(256) void minibatch_step_kernel(MinibatchStepArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int kArena = 2 * (256 + 256) * kRowBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t arena[kArena];
  __shared__ int32_t s_up[1025], s_dn[1025], s_wsum[4];
  const int tid = threadIdx.x;
  const GroupedGemmArgs& gu = a.up;
  const int P = gu.offsets[gu.eb + gu.E_loc];  // local rows
  const int u0 = min(a.up0, P), u1 = min(a.up1, P);
  const int d0 = min(a.dn0, P), d1 = min(a.dn1, P);
  const int c0 = min(a.cp0, P), c1 = min(a.cp1, P);
  range_tile_prefix<256>(gu, u0, u1, s_up, s_wsum);
  range_tile_prefix<256>(a.down, d0, d1, s_dn, s_wsum);
  const int ntn_up = (gu.F + 127) / 128, ntn_dn = (gu.d + 255) / 256;
  const int n_cp = (c1 - c0 + kCopyRows - 1) / kCopyRows;
  const int n_up = s_up[gu.E_loc] * ntn_up;
  const int n_dn = s_dn[gu.E_loc] * ntn_dn;
  const int total = n_cp + n_up + n_dn;
  const int G_ = gridDim.x;
  const int vb = (G_ % 8 == 0) ? (blockIdx.x % 8) * (G_ / 8) + blockIdx.x / 8 : blockIdx.x;
  for (int t = vb; t < total; t += G_) {
    if (t < n_cp) {
      // mover task: rows [c0 + t*16, ...) of the next minibatch into its slot
      const int d = gu.d, nv = d / 8;
      const int rb = c0 + t * kCopyRows, re = min(rb + kCopyRows, c1);
      for (int v = tid; v < (re - rb) * nv; v += 256) {
        const int r = rb + v / nv, c = v % nv;
        const int tok = a.pair_of_row[r] / a.k;
        const u32x4_t val = reinterpret_cast<const u32x4_t*>((const bf16_t*)a.x + (int64_t)tok * d)[c];
        reinterpret_cast<u32x4_t*>((bf16_t*)a.ring_dst + (int64_t)(r - c0) * d)[c] = val;
      }
    } else if (t < n_cp + n_up) {
      int e_loc, row0, row_end, n0;
      range_tile(gu, s_up, ntn_up, 256, u0, u1, t - n_cp, e_loc, row0, row_end, n0, 128);
      gemm_tile<KIND_UP, 256, 128>(gu, arena, __builtin_amdgcn_readfirstlane(e_loc),
                                   __builtin_amdgcn_readfirstlane(row0), __builtin_amdgcn_readfirstlane(row_end), 0,
                                   __builtin_amdgcn_readfirstlane(n0), 0);
    } else {
      int e_loc, row0, row_end, n0;
      range_tile(a.down, s_dn, ntn_dn, 256, d0, d1, t - n_cp - n_up, e_loc, row0, row_end, n0, 256);
      gemm_tile<KIND_DOWN, 256, 256>(a.down, arena, __builtin_amdgcn_readfirstlane(e_loc),
                                     __builtin_amdgcn_readfirstlane(row0), __builtin_amdgcn_readfirstlane(row_end), 0,
                                     __builtin_amdgcn_readfirstlane(n0), 0);
    }
  }
#endif
}

hipError_t launch_minibatch_step(const MinibatchStepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(minibatch_step_kernel, dim3(256), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mok
