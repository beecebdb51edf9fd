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
// Tiling: a workgroup of NW waves (four as 2 x 2, or eight as 4 x 2 or
// 2 x 4; the choice per kind is in gemm_bf16() below) computes a BM x BN
// tile (per B matrix; UP computes the W1 and W3 tiles of the same columns),
// each wave a block of 32x32 MFMA tiles.  K advances in stages of BK (32 or
// 64) through a ring of NS LDS stage buffers (per kind, below), so NS - 1
// stages are in flight while one is multiplied.  Every
// operand goes from HBM straight to LDS
// (buffer_load_dwordx4 ... lds, 1 KB per wave instruction, no VGPRs),
// through buffer resources rebased on the tile so that rows past the data
// read as zero, in the layout it has in memory:
//   K-contiguous operands ([row][k]): LDS rows of BK * 2 bytes in 16-byte
//     chunks, XOR-swizzled; fragments are 16-byte reads (ds_read_b128).
//   M- or N-contiguous operands ([k][row], the backward products): LDS rows
//     of one k, 64-byte chunks XOR-swizzled by k; fragments are transposing
//     reads (ds_read_b64_tr_b16), which hand each lane four consecutive k of
//     one row, so no transpose pass through registers is needed.
// The swizzles make fragment reads bank-conflict free.  Fragments of the
// next 16-K slice are read while the MFMAs of the current one run; the one
// workgroup barrier per stage sits between the two MFMA halves of a stage.
//
// Scheduling: row-grouped kinds run a persistent loop over the tiles of all
// local experts in (expert, n-tile, m-tile) order, with the tile prefix of
// each expert computed on the device by the counting sort, so the host never
// needs the data-dependent row count.  Workgroup b runs on XCD b mod 8; the
// loop hands each XCD a contiguous run of tiles so that m-tiles sharing a
// weight tile meet in one L2.  The first stages of the next tile are loaded
// while the current tile's epilogue runs.  Every output element is produced
// by one workgroup with a fixed K order: results are run-to-run identical
// (no split-K, no float atomics).
#include "mok_device.h"
#include "mok_internal.h"
#include "gemm_common.h"
#include "gemm_pipe.h"

// Non-temporal copies of the GEMM operands, per kind family and operand: the
// weight-gradient GEMMs' B copies (X rows for dW1/dW3, H rows for dW2) carry
// the hint.  Measured on dW1/dW3: 2.6-2.8 ms with the hint on B (or on A, or
// both) against 3.0-3.1 ms without; dW2 is unaffected.  The row kinds keep
// their weight and row tiles in L2 for the other tiles that share them: the
// hint on either operand makes UP and DOWN 10-35 % slower.
// Row tiles: skip the MFMAs of 32-row blocks wholly past the expert's end.
#ifndef MOK_SKIP_PAD
#define MOK_SKIP_PAD 1
#endif
#ifndef MOK_ROW_GM
#define MOK_ROW_GM 4  // m-tiles per raster group of the row-grouped kinds (tile_mn)
#endif
#ifndef MOK_DW_NT_A
#define MOK_DW_NT_A 0
#endif
#ifndef MOK_DW_NT_B
#define MOK_DW_NT_B 1
#endif
#ifndef MOK_ROW_NT_A
#define MOK_ROW_NT_A 0
#endif
// Non-temporal fp32 weight-gradient stores, per kind (same-box A/B at T 8192,
// d 4096, E 128, k 8, F 1536, three alternating rounds: dW1/dW3 2.73-2.74 ->
// 2.67-2.71 ms with the hint, training step 10.58-10.65 -> 10.53-10.63 ms;
// dW2 1.42 -> 1.47-1.49 ms with it, so dW2 keeps the default policy).
#ifndef MOK_DW2_NT_STORE
#define MOK_DW2_NT_STORE 0
#endif
#ifndef MOK_DW13_NT_STORE
#define MOK_DW13_NT_STORE 1
#endif
#ifndef MOK_ROW_NT_B
#define MOK_ROW_NT_B 0
#endif

namespace mok {


typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// One operand's share of an LDS stage: ROWS tile rows (M or N) by BK, copied
// by NW waves.
template <bool MN, int ROWS, int BK, int NW>
struct OpGeo {
  static constexpr int BYTES = ROWS * BK * 2;     // per stage
  static constexpr int INST = BYTES / 1024 / NW;  // DMA instructions per wave per stage
  static constexpr int ROWB = ROWS * 2;          // MN: bytes of one k row
  static constexpr int LPR = ROWS / 8;           // MN: lanes per k row in a DMA instruction
  static constexpr int RPI = 64 / LPR;           // MN: k rows per DMA instruction
  static constexpr int KLPR = BK / 8;            // K-contiguous: lanes per row in a DMA instruction
  static constexpr int KRPI = 64 / KLPR;         // K-contiguous: rows per DMA instruction
  static_assert(INST >= 1 && BYTES % (1024 * NW) == 0, "stage share must fill whole wave DMA instructions");
  static_assert(!MN || (ROWS % 128 == 0 && RPI >= 1), "M/N-contiguous tile rows");
};

// One output tile: its DMA sources, K loop and epilogue, with NS LDS stage
// buffers of BK (32 or 64) K values, computed by NW waves, WMW along M and
// NW / WMW along N.  NW = 4 (2 x 2): 128 x 128 per wave, 256 accumulators.
// NW = 8, two waves per SIMD with 128 accumulators each, so that one wave's
// MFMAs run while the other waits to issue its copies or for its fragments:
// 4 x 2 (64 x 128 per wave; each B fragment is read by four waves) or 2 x 4
// (128 x 64; each A fragment read by four), the latter for kinds whose B
// fragments come from the slower transposing LDS reads.
// All members are wave-uniform except the per-lane DMA offsets.
template <int KIND, int BM, int BN, int NS, int BK, int NW = 4, int WMW = 2>
struct TileJob {
  using Tr = Traits<KIND>;
  static constexpr int NB = Tr::NB, BROWS = NB * BN, WNW = NW / WMW;
  static constexpr int TM = BM / WMW, TN = BN / WNW, FM = TM / 32, FN = TN / 32;
  static_assert(FM >= 1 && FN >= 1 && (FN % 2 == 0 || NB == 2 || Tr::GROUP_K), "wave tile");
  using GA = OpGeo<Tr::A_MN, BM, BK, NW>;
  using GB = OpGeo<Tr::B_MN, BROWS, BK, NW>;
  static constexpr int KK = BK / 16;  // 16-K MFMA slices per stage
  // Epilogue staging per wave: a round of 32 rows (8 KB), or of 16 rows (4 KB)
  // for the eight-wave row kinds with 64-K stages (two stages of 64 KB leave
  // 32 KB for the staging).
  static constexpr int HR = (!Tr::GROUP_K && NW == 8 && BK == 64) ? 16 : 32;
  static constexpr int EP_BYTES = HR * 256;
  static_assert(BK == 32 || BK == 64, "stage depth");
  static constexpr int A_BYTES = GA::BYTES;
  static constexpr int STAGE = GA::BYTES + GB::BYTES;
  static constexpr int D = GA::INST + GB::INST;  // DMA instructions per wave per stage
  // Weight-gradient kinds stage their fp32 epilogue in the stage buffers;
  // the row kinds' callers give them a staging area of NW * EP_BYTES.
  static_assert(!Tr::GROUP_K || STAGE / 4 >= 8192, "epilogue staging needs 8 KB per wave");
  static_assert(NS >= 2 && NS <= 5 && (NS - 1) * D <= 63, "stage count (vmcnt holds at most 63)");
  static_assert(!(NB == 2 && Tr::B_MN), "paired B matrices are K-contiguous");
  // Which operand copies carry the non-temporal hint (see the macros above).
  static constexpr bool kNtA = Tr::GROUP_K ? MOK_DW_NT_A : MOK_ROW_NT_A;
  static constexpr bool kNtB = Tr::GROUP_K ? MOK_DW_NT_B : MOK_ROW_NT_B;

  struct Frags {
    bf16x8_t a[FM];
    bf16x8_t b[NB][FN];
  };
  // DH epilogue operands of one round (the saved A and B at this lane's four
  // 8-column pieces), loaded a round ahead.
  struct SavedAB {
    u32x4_t a[4], b[4];
  };

  const GroupedGemmArgs* args;
  GemmGeom G;
  TileCoord c;
  int wid, lane, wm, wn;
  int kbeg, kend, nk;
  int nvb;  // this wave's 32-row blocks that hold rows of the expert (the rest: no MFMAs)
  i32x4_t rsA, rsB0, rsB1;  // K-contiguous sources (whole tile)
  uint32_t offA[GA::INST], offB[GB::INST];

  __device__ __forceinline__ void init(const GroupedGemmArgs& a, const TileCoord& tc) {
    args = &a;
    G = geom_of<KIND>(a.d, a.F);
    c = tc;
    lane = threadIdx.x & 63;
    wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    wm = wid / WNW;
    wn = wid % WNW;
    kbeg = Tr::GROUP_K ? c.row0 : 0;
    kend = Tr::GROUP_K ? c.row_end : G.K;
    nk = (kend - kbeg + BK - 1) / BK;
    nvb = FM;
    if constexpr (!Tr::GROUP_K && MOK_SKIP_PAD && NW == 8) {  // (256 accumulators: the branches spill)
      // rows past the expert's end are zero padding and are never stored:
      // their MFMAs are skipped (less work, less power)
      const int left = c.row_end - (c.row0 + wm * TM);
      nvb = left <= 0 ? 0 : (left >= TM ? FM : (left + 31) / 32);
    }
    const bf16_t* Abase = (const bf16_t*)a.A;
    rsA = rsB0 = rsB1 = make_rsrc(Abase, 0u);
    // ---- A
    if constexpr (!Tr::A_MN) {
      const int rows = c.row_end - c.row0 < BM ? c.row_end - c.row0 : BM;
      if (a.gather_rows) {
        // pull dispatch: each row comes straight from its token's row of x
        rsA = make_rsrc(Abase, (uint32_t)(a.gather_src_rows * G.lda * 2));
#pragma unroll
        for (int q = 0; q < GA::INST; ++q) {
          const int r = (wid * GA::INST + q) * GA::KRPI + lane / GA::KLPR;
          const int tok = r < rows ? a.gather_rows[c.row0 + r] / a.k_top : -1;
          offA[q] = tok >= 0 ? (uint32_t)(tok * G.lda * 2 + swz_k<BK>(r, lane % GA::KLPR) * 16) : 0xFFFFFFF0u;
        }
      } else {
        rsA = make_rsrc(Abase + ((int64_t)c.row0 - a.a_row_shift) * G.lda, (uint32_t)((int64_t)rows * G.lda * 2));
#pragma unroll
        for (int q = 0; q < GA::INST; ++q) {
          const int r = (wid * GA::INST + q) * GA::KRPI + lane / GA::KLPR;
          offA[q] = (uint32_t)(r * G.lda * 2 + swz_k<BK>(r, lane % GA::KLPR) * 16);
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < GA::INST; ++q) {
        const int r = (wid * GA::INST + q) * GA::RPI + lane / GA::LPR;  // k row in the stage
        const int p = lane % GA::LPR;
        const int col = swz_mn(r, p >> 2) * 32 + (p & 3) * 8;           // logical column of this 16 B
        offA[q] = (uint32_t)((r * G.lda + col) * 2);
      }
    }
    // ---- B
    if constexpr (!Tr::B_MN) {
      const int nb_rows = G.N - c.n0 < BN ? G.N - c.n0 : BN;
      const bf16_t* b0 = (const bf16_t*)a.B0 + (int64_t)c.e_loc * G.b_estride + (int64_t)c.n0 * G.ldb;
      rsB0 = make_rsrc(b0, (uint32_t)((int64_t)nb_rows * G.ldb * 2));
      if constexpr (NB == 2) {
        const bf16_t* b1 = (const bf16_t*)a.B1 + (int64_t)c.e_loc * G.b_estride + (int64_t)c.n0 * G.ldb;
        rsB1 = make_rsrc(b1, (uint32_t)((int64_t)nb_rows * G.ldb * 2));
      }
#pragma unroll
      for (int q = 0; q < GB::INST; ++q) {
        const int r = (wid * GB::INST + q) * GB::KRPI + lane / GB::KLPR;  // LDS row
        const int rl = (NB == 2 && r >= BN) ? r - BN : r;                 // row within its matrix
        offB[q] = (uint32_t)(rl * G.ldb * 2 + swz_k<BK>(r, lane % GB::KLPR) * 16);
      }
    } else {
#pragma unroll
      for (int q = 0; q < GB::INST; ++q) {
        const int r = (wid * GB::INST + q) * GB::RPI + lane / GB::LPR;
        const int p = lane % GB::LPR;
        const int col = swz_mn(r, p >> 2) * 32 + (p & 3) * 8;
        offB[q] = Tr::GROUP_K && a.gather_rows ? (uint32_t)(col * 2) : (uint32_t)((r * G.ldb + col) * 2);
      }
    }
  }

  // Issue the copies of stage s into LDS stage buffer s % NS.
  __device__ __forceinline__ void issue(int s, uint8_t* arena) const { issue_part<0, D>(s, arena); }

  // The first NS stages.
  __device__ __forceinline__ void prologue(uint8_t* arena) const {
    for (int s = 0; s < NS && s < nk; ++s) issue(s, arena);
  }

  // Copies [Q0, Q1) of the D of a stage (A's first, then B's), so that a
  // stage's copies can be spread between MFMAs.
  template <int Q0, int Q1>
  __device__ __forceinline__ void issue_part(int s, uint8_t* arena) const {
    constexpr int QB = GA::INST;  // index of the first B copy
    uint8_t* st = arena + (s % NS) * STAGE;
    const int k0 = kbeg + s * BK;
    if constexpr (Q0 >= QB) {
      // no A copies in this part
    } else if constexpr (!Tr::A_MN) {
#pragma unroll
      for (int q = Q0; q < (Q1 < QB ? Q1 : QB); ++q)
        dma_b128<kNtA>(rsA, lds_addr(st + (wid * GA::INST + q) * 1024), offA[q], k0 * 2);
    } else {
      // rows [k0, kend) of columns [m0, ...) of this expert's rows; rows past kend read zero
      const int64_t col0 = c.m0 + (KIND == KIND_DW13 ? (int64_t)c.z * args->F : 0);
      const bf16_t* p = (const bf16_t*)args->A + (int64_t)k0 * G.lda + col0;
      const int64_t bytes = ((int64_t)(kend - k0) * G.lda - col0) * 2;
      const i32x4_t rs = make_rsrc(p, bytes > 0 ? (uint32_t)bytes : 0u);
#pragma unroll
      for (int q = Q0; q < (Q1 < QB ? Q1 : QB); ++q)
        dma_b128<kNtA>(rs, lds_addr(st + (wid * GA::INST + q) * 1024), offA[q], 0);
    }
    uint8_t* sb = st + A_BYTES;
    constexpr int B0q = Q0 > QB ? Q0 - QB : 0, B1q = Q1 > QB ? Q1 - QB : 0;  // this part's B copies
    if constexpr (B1q <= B0q) {
      // no B copies in this part
    } else if constexpr (!Tr::B_MN) {
#pragma unroll
      for (int q = B0q; q < B1q; ++q)
        dma_b128<kNtB>((NB == 2 && (wid * GB::INST + q) * GB::KRPI >= BN) ? rsB1 : rsB0,
                 lds_addr(sb + (wid * GB::INST + q) * 1024), offB[q], k0 * 2);
    } else if constexpr (!Tr::GROUP_K) {
      // weights [K][N] of this expert; DX takes k < F from W1 and the rest from W3
      const bool second = k0 >= G.ksplit;
      const int kl = second ? k0 - G.ksplit : k0;
      const bf16_t* base = (const bf16_t*)(second ? args->B1 : args->B0) + (int64_t)c.e_loc * G.b_estride;
      const int krows = second ? G.K - G.ksplit : G.ksplit;
      const bf16_t* p = base + (int64_t)kl * G.ldb + c.n0;
      const int64_t bytes = ((int64_t)(krows - kl) * G.ldb - c.n0) * 2;
      const i32x4_t rs = make_rsrc(p, bytes > 0 ? (uint32_t)bytes : 0u);
#pragma unroll
      for (int q = B0q; q < B1q; ++q) dma_b128<kNtB>(rs, lds_addr(sb + (wid * GB::INST + q) * 1024), offB[q], 0);
    } else if (!args->gather_rows) {
      const bf16_t* p = (const bf16_t*)args->B0 + (int64_t)k0 * G.ldb + c.n0;
      const int64_t bytes = ((int64_t)(kend - k0) * G.ldb - c.n0) * 2;
      const i32x4_t rs = make_rsrc(p, bytes > 0 ? (uint32_t)bytes : 0u);
#pragma unroll
      for (int q = B0q; q < B1q; ++q) dma_b128<kNtB>(rs, lds_addr(sb + (wid * GB::INST + q) * 1024), offB[q], 0);
    } else {
      // B rows are token rows of x: row k of the expert is x[gather_rows[k] / k_top]
      static_assert(GB::RPI == 2, "gathered rows: two k rows per DMA instruction");
      const i32x4_t rs = make_rsrc(args->B0, (uint32_t)(args->gather_src_rows * G.ldb * 2));
#pragma unroll
      for (int q = B0q; q < B1q; ++q) {
        const int kr = k0 + (wid * GB::INST + q) * 2;
        int32_t i0 = -1, i1 = -1;
        if (kr < kend) sload_pair(args->gather_rows + kr, kr + 1 < kend, i0, i1);
        i1 = kr + 1 < kend ? i1 : -1;
        const int32_t pr = (lane >> 5) ? i1 : i0;
        const uint32_t off =
            pr >= 0 ? (uint32_t)(((int64_t)(pr / args->k_top) * G.ldb + c.n0) * 2) + offB[q] : 0xFFFFFFF0u;
        dma_b128<kNtB>(rs, lds_addr(sb + (wid * GB::INST + q) * 1024), off, 0);
      }
    }
  }

  // Fragment of tile rows [rb, rb + 32) from an M/N-contiguous stage: lane l
  // gets k = 16 kk + 8 (l / 32) + 0..7 of row rb + l % 32.  In each group of
  // 16 lanes, lane j names four consecutive values of k row j / 4 (columns
  // 4 (j % 4) + 0..3 of the group's 16) and the transposing read returns to
  // lane j the values of column j from k rows 0..3.
  template <int ROWB>
  __device__ __forceinline__ bf16x8_t read_tr(const uint8_t* base, int rb, int kk) const {
    const int g = lane >> 4, jj = lane & 15;
    const int kr = kk * 16 + 8 * (g >> 1) + (jj >> 2);
    const int col = rb + 16 * (g & 1) + 4 * (jj & 3);
    const uint8_t* p0 = base + kr * ROWB + swz_mn(kr, col >> 5) * 64 + (col & 31) * 2;
    const i16x4_t lo =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(const __attribute__((address_space(3))) void*)p0);
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4_t*)(const __attribute__((address_space(3))) void*)(p0 + 4 * ROWB));
    const i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
  }

  // Fragments of 16-K slice kk (0 or 1) of the stage in buffer `buf`.
  __device__ __forceinline__ void read(int buf, int kk, const uint8_t* arena, Frags& f) const {
    const uint8_t* st = arena + buf * STAGE;
    if constexpr (!Tr::A_MN) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * TM + i * 32 + (lane & 31);
        f.a[i] = *reinterpret_cast<const bf16x8_t*>(st + r * (BK * 2) + swz_k<BK>(r, kk * 2 + (lane >> 5)) * 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i) f.a[i] = read_tr<GA::ROWB>(st, wm * TM + i * 32, kk);
    }
    const uint8_t* sb = st + A_BYTES;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int rb = b * BN + wn * TN + j * 32;
        if constexpr (!Tr::B_MN) {
          const int r = rb + (lane & 31);
          f.b[b][j] = *reinterpret_cast<const bf16x8_t*>(sb + r * (BK * 2) + swz_k<BK>(r, kk * 2 + (lane >> 5)) * 16);
        } else {
          f.b[b][j] = read_tr<GB::ROWB>(sb, rb, kk);
        }
      }
  }

  __device__ __forceinline__ void mma(f32x16_t (&acc)[NB][FM][FN], const Frags& f) const { mma_part<0, 1>(acc, f); }

  // MFMAs [g, g + 1) / NG of a slice, in (b, i, j) order.
  template <int g, int NG>
  __device__ __forceinline__ void mma_part(f32x16_t (&acc)[NB][FM][FN], const Frags& f) const {
    constexpr int TOT = NB * FM * FN, L0 = g * TOT / NG, L1 = (g + 1) * TOT / NG;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int L = (b * FM + i) * FN + j;
          if (L >= L0 && L < L1 && i < nvb)
            acc[b][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[b][j], acc[b][i][j], 0, 0, 0);
        }
  }

  // The last slice of a stage with the next stage's copies spread between
  // its MFMAs (four groups).
  template <int G>
  __device__ __forceinline__ void mma_issue(f32x16_t (&acc)[NB][FM][FN], const Frags& f, bool copy, int s,
                                            uint8_t* arena) const {
    if constexpr (G < 4) {
      if (copy) issue_part<G * D / 4, (G + 1) * D / 4>(s, arena);
      __builtin_amdgcn_sched_barrier(0);
      mma_part<G, 4>(acc, f);
      __builtin_amdgcn_sched_barrier(0);
      mma_issue<G + 1>(acc, f, copy, s, arena);
    }
  }

  // K loop.  On entry the copies of stages 0 .. min(nk, NS) - 1 have been
  // issued in order; on exit every stage has been read by this wave (the
  // caller meets the workgroup before reusing the buffers).
  __device__ __forceinline__ void mainloop(f32x16_t (&acc)[NB][FM][FN], uint8_t* arena) const {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[b][i][j][r] = 0.f;
    if (nk <= 0) return;
    wait_stages<D, NS - 1>(nk - 1 < NS - 1 ? nk - 1 : NS - 1);  // stages issued after stage 0
    // (sched_barrier: keep each batch of fragment reads ahead of the MFMAs
    // that hide its latency; the scheduler would otherwise sink them).
    // Slice kk of a stage sits in fa for even kk and in fb for odd kk.
    Frags fa, fb;
    read(0, 0, arena, fa);
    for (int kt = 0; kt + 1 < nk; ++kt) {
#pragma unroll
      for (int kk = 0; kk + 1 < KK; ++kk) {
        read(kt % NS, kk + 1, arena, (kk & 1) ? fa : fb);
        __builtin_amdgcn_sched_barrier(0);
        mma(acc, (kk & 1) ? fb : fa);
      }
      // stage kt + 1 landed (the NS - 2 after it may still fly), and every
      // wave is done with stage kt, whose buffer takes stage kt + NS
      wait_stages<D, NS - 2>(nk - 2 - kt < NS - 2 ? nk - 2 - kt : NS - 2);
      read((kt + 1) % NS, 0, arena, fa);
      mma_issue<0>(acc, fb, kt + NS < nk, kt + NS, arena);  // slice KK - 1 (KK is even)
    }
    // last stage (peeled: its last slice follows no barrier)
#pragma unroll
    for (int kk = 0; kk + 1 < KK; ++kk) {
      read((nk - 1) % NS, kk + 1, arena, (kk & 1) ? fa : fb);
      mma(acc, (kk & 1) ? fb : fa);
    }
    mma(acc, fb);
  }

  // Epilogue.  bf16 outputs go through this wave's own 8 KB of `staging`
  // (32 KB for the workgroup): 16-byte row-contiguous stores.  fp32 weight
  // gradients are stored straight from the accumulators: each half-wave
  // writes 32 consecutive floats of one row, a whole 128-byte line (measured
  // faster than 16-byte stores from transposed accumulators, whose
  // instructions each touch 32 rows).
  // Saved A and B of DH epilogue round (i, jp); rows past the expert read as zero.
  __device__ __forceinline__ void load_saved(int i, int jp, SavedAB& p) const {
    const GroupedGemmArgs& a = *args;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int seg = q * 64 + lane;
      const int row = c.row0 + wm * TM + i * 32 + (seg >> 3), col = c.n0 + wn * TN + jp * 64 + (seg & 7) * 8;
      const bool ok = row < c.row_end && col < G.N;
      const int64_t o = ok ? (int64_t)row * G.N + col : 0;
      p.a[q] = ok ? *reinterpret_cast<const u32x4_t*>((const bf16_t*)a.save_a + o) : u32x4_t{0u, 0u, 0u, 0u};
      p.b[q] = ok ? *reinterpret_cast<const u32x4_t*>((const bf16_t*)a.save_b + o) : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  // First round's epilogue loads, issued before the next tile's copies so
  // that waiting for them does not wait for those copies too.
  __device__ __forceinline__ void epilogue_prefetch(SavedAB& p0) const {
    if constexpr (KIND == KIND_DH) load_saved(0, 0, p0);
  }

  __device__ __forceinline__ void epilogue(const f32x16_t (&acc)[NB][FM][FN], uint8_t* staging,
                                           SavedAB& p0) const {
    SavedAB p1;
    float* ep = reinterpret_cast<float*>(staging + wid * EP_BYTES);
    const GroupedGemmArgs& a = *args;
    const int wrow0 = wm * TM, wcol0 = wn * TN;
    if constexpr (Tr::GROUP_K) {
      // M and N are multiples of 32: a 32 x 32 block is wholly in or out
      float* outp = (float*)(KIND == KIND_DW13 && c.z ? a.out1 : a.out0) + (int64_t)c.e_loc * G.M * G.N;
      float* lp = outp + (int64_t)(c.m0 + wrow0 + (lane >> 5) * 4) * G.N + c.n0 + wcol0 + (lane & 31);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if (c.m0 + wrow0 + i * 32 >= G.M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if (c.n0 + wcol0 + j * 32 >= G.N) continue;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float* q = lp + (int64_t)(i * 32 + (r >> 2) * 8 + (r & 3)) * G.N + j * 32;
            if constexpr (KIND == KIND_DW13 ? MOK_DW13_NT_STORE : MOK_DW2_NT_STORE)
              __builtin_nontemporal_store(acc[0][i][j][r], q);
            else *q = acc[0][i][j][r];
          }
        }
      }
    } else if constexpr (NB == 2) {
      // UP: gate (W1) and up (W3) accumulators of one HR x 32 block per round
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int hf = 0; hf < 32 / HR; ++hf) {
#pragma unroll
          for (int r = hf * HR / 2; r < (hf + 1) * HR / 2; ++r) {
            const int rr = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3) - hf * HR;
            ep[rr * 32 + (lane & 31)] = acc[0][i][j][r];
            ep[HR * 32 + rr * 32 + (lane & 31)] = acc[1][i][j][r];
          }
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int q = 0; q < HR / 16; ++q) {
            const int seg = q * 64 + lane;
            const int rr = seg >> 2, c8 = (seg & 3) * 8;
            const int row = c.row0 + wrow0 + i * 32 + hf * HR + rr, col = c.n0 + wcol0 + j * 32 + c8;
            if (row < c.row_end && col < G.N) {
              const f32x4_t* pv = reinterpret_cast<const f32x4_t*>(&ep[rr * 32 + c8]);
              const f32x4_t* pu = reinterpret_cast<const f32x4_t*>(&ep[HR * 32 + rr * 32 + c8]);
              const f32x4_t v0 = pv[0], v1 = pv[1], u0 = pu[0], u1 = pu[1];
              const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
              const float u[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
              u32x4_t h, av, bv;
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const float h0 = v[2 * t] * sigmoidf_(v[2 * t]) * u[2 * t];
                const float h1 = v[2 * t + 1] * sigmoidf_(v[2 * t + 1]) * u[2 * t + 1];
                h[t] = (uint32_t)f2bf(h0) | ((uint32_t)f2bf(h1) << 16);
                av[t] = (uint32_t)f2bf(v[2 * t]) | ((uint32_t)f2bf(v[2 * t + 1]) << 16);
                bv[t] = (uint32_t)f2bf(u[2 * t]) | ((uint32_t)f2bf(u[2 * t + 1]) << 16);
              }
              const int64_t o = (int64_t)row * G.N + col;
              *reinterpret_cast<u32x4_t*>((bf16_t*)a.out0 + o) = h;
              if (a.save) {
                *reinterpret_cast<u32x4_t*>((bf16_t*)a.save_a + o) = av;
                *reinterpret_cast<u32x4_t*>((bf16_t*)a.save_b + o) = bv;
              }
            }
          }
          __builtin_amdgcn_wave_barrier();
        }
    } else {
      // one HR x 64 block per round (DH: HR = 32)
      static_assert(KIND != KIND_DH || HR == 32, "DH prefetches whole 32-row rounds");
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jp = 0; jp < FN / 2; ++jp)
#pragma unroll
        for (int hf = 0; hf < 32 / HR; ++hf) {
          const int t = i * (FN / 2) + jp;  // round
          SavedAB& cur = (t & 1) ? p1 : p0;
          if constexpr (KIND == KIND_DH) {
            if (t + 1 < FM * (FN / 2)) load_saved((t + 1) / (FN / 2), (t + 1) % (FN / 2), (t & 1) ? p0 : p1);
          }
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int r = hf * HR / 2; r < (hf + 1) * HR / 2; ++r) {
              const int rr = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3) - hf * HR;
              ep[rr * 64 + jj * 32 + (lane & 31)] = acc[0][i][2 * jp + jj][r];
            }
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int q = 0; q < HR / 8; ++q) {
            const int seg = q * 64 + lane;
            const int rr = seg >> 3, c8 = (seg & 7) * 8;
            const f32x4_t* pv = reinterpret_cast<const f32x4_t*>(&ep[rr * 64 + c8]);
            const f32x4_t v0 = pv[0], v1 = pv[1];
            const int col = c.n0 + wcol0 + jp * 64 + c8;
            {
              const int row = c.row0 + wrow0 + i * 32 + hf * HR + rr;
              if (row < c.row_end && col < G.N) {
                const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                const int64_t o = (int64_t)row * G.N + col;
                if constexpr (KIND == KIND_DH) {
                  const u32x4_t av = cur.a[q], bv = cur.b[q];
                  u32x4_t da, db;
#pragma unroll
                  for (int t = 0; t < 4; ++t) {
                    float dav[2], dbv[2];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                      const float x1 = __uint_as_float(hh ? (av[t] & 0xFFFF0000u) : (av[t] << 16));
                      const float x3 = __uint_as_float(hh ? (bv[t] & 0xFFFF0000u) : (bv[t] << 16));
                      const float sg = sigmoidf_(x1);
                      const float dh = v[2 * t + hh];
                      dav[hh] = dh * x3 * sg * (1.0f + x1 * (1.0f - sg));
                      dbv[hh] = dh * x1 * sg;
                    }
                    da[t] = (uint32_t)f2bf(dav[0]) | ((uint32_t)f2bf(dav[1]) << 16);
                    db[t] = (uint32_t)f2bf(dbv[0]) | ((uint32_t)f2bf(dbv[1]) << 16);
                  }
                  bf16_t* dab = (bf16_t*)a.out0 + (int64_t)row * 2 * a.F;
                  *reinterpret_cast<u32x4_t*>(dab + col) = da;
                  *reinterpret_cast<u32x4_t*>(dab + a.F + col) = db;
                } else {
                  u32x4_t y;
#pragma unroll
                  for (int t = 0; t < 4; ++t)
                    y[t] = (uint32_t)f2bf(v[2 * t]) | ((uint32_t)f2bf(v[2 * t + 1]) << 16);
                  *reinterpret_cast<u32x4_t*>((bf16_t*)a.out0 + o) = y;
                }
              }
            }
          }
          __builtin_amdgcn_wave_barrier();
        }
    }
  }
};

// Persistent grouped GEMM.  LDS: the NS stage buffers, then either the bf16
// epilogue staging area (row kinds; 4 or 8 KB per wave) or the mailbox through
// which wave 0 hands the tile taken from the queue to the workgroup
// (weight-gradient kinds).  The tile-prefix table is searched in global
// memory through the scalar cache.
template <int KIND, int BM, int BN, int NS, int BK, int NW, int WMW>
__global__ __launch_bounds__(NW * 64) void grouped_gemm_bf16_kernel(GroupedGemmArgs args) {
#if defined(__HIP_DEVICE_COMPILE__)  // device-only builtins; the host pass needs only the launch stub
  using Tr = Traits<KIND>;
  using Job = TileJob<KIND, BM, BN, NS, BK, NW, WMW>;
  constexpr int kExtra = Tr::GROUP_K ? 256 : NW * Job::EP_BYTES;
  static_assert(NS * Job::STAGE + kExtra <= 163840, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t arena[NS * Job::STAGE + kExtra];
  uint8_t* const staging = arena + NS * Job::STAGE;
  int* const mbox = reinterpret_cast<int*>(staging);

  const GemmGeom G = geom_of<KIND>(args.d, args.F);
  const int tid = threadIdx.x;
  const int E_loc = args.E_loc;
  const int ntn = (G.N + BN - 1) / BN;
  const int xcd = blockIdx.x % 8;
  constexpr int NZ = KIND == KIND_DW13 ? 2 : 1;  // DW13 computes dW1 (z = 0) and dW3 (z = 1)
  const int32_t* tp = args.tile_prefix + ((BM == 64) ? 0 : (BM == 128 ? 1 : 2)) * (E_loc + 1);

  // Weight-gradient kinds: the heaviest-first tile sequence (expert-major,
  // T tiles per expert) is cut into eight runs; bound(x) is the start of run
  // x, the first tile whose cumulative work reaches x eighths of the total.
  const int ntm_k = Tr::GROUP_K ? (G.M + BM - 1) / BM : 0;
  const int T = NZ * ntm_k * ntn;
  const int32_t* rk = args.expert_order;  // per rank {expert, row0, row_end, work prefix}
  auto bound = [&](int x) -> int {
    if (x <= 0 || E_loc == 0) return 0;
    if (x >= 8) return E_loc * T;
    const int64_t target = (int64_t)T * sload(rk + 4 * E_loc + 3) * x / 8;
    int lo = 0, hi = E_loc - 1;  // last rank whose tiles start at or before target
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)T * sload(rk + 4 * mid + 3) <= target) lo = mid; else hi = mid - 1;
    }
    const int w0 = sload(rk + 4 * lo + 3), w1 = sload(rk + 4 * lo + 7);
    const int64_t j = (target - (int64_t)T * w0) / (w1 - w0);  // whole tiles of rank lo by target
    return lo * T + (int)(j < T ? j : T);
  };
  int total, tbeg = 0;
  if constexpr (!Tr::GROUP_K) {
    total = sload(tp + E_loc) * ntn;
  } else {
    tbeg = bound(xcd);
    total = bound(xcd + 1) - tbeg;
  }
  // Row-grouped kinds: equal-sized tiles in a static round-robin.  XCD-aware
  // order: workgroup b (on XCD b % 8) takes tiles from the contiguous run
  // [x * G/8, (x+1) * G/8) of each round of G tiles.  Weight-gradient kinds:
  // the work of a tile grows with its expert's rows, so the tiles are taken
  // heaviest expert first (rank order of the counting sort), the sequence is
  // cut into 8 runs of equal work and the workgroups of XCD x pull run x's
  // tiles from counter x: an expert's tiles mostly share one L2, and an
  // expert heavier than an eighth of the work spreads over several XCDs.
  // A workgroup whose run is exhausted goes on to the runs of the next
  // XCDs in turn (x + 1, x + 2, ... mod 8), so that the tail of a run of
  // long tiles is shared out instead of keeping the other XCDs waiting.
  // Each tile is still computed whole by one workgroup, so the results do
  // not depend on the assignment.
  const int G_ = gridDim.x;
  const int vb = (G_ % 8 == 0) ? xcd * (G_ / 8) + blockIdx.x / 8 : blockIdx.x;
  // Weight-gradient kinds: thread 0 takes the tile after the current one from
  // the queue as the current one starts, so the atomic's latency is hidden.
  // vx is the XCD whose run is being taken, [vbeg, vbeg + vcnt) that run.
  int taken = 0, vx = xcd, vbeg = tbeg, vcnt = total, hops = 0;
  auto take = [&]() {
    if constexpr (Tr::GROUP_K) {
      if (tid == 0) taken = atomicAdd(args.queue + vx, 1);
    }
  };
  // Position in the heaviest-first sequence of the v-th tile taken from run
  // vx, moving on to the next runs while v is past the end; -1 once all
  // eight runs are exhausted.  Called by every wave with the same v, right
  // after the mailbox has been read.
  auto resolve = [&](int v) -> int {
    if constexpr (Tr::GROUP_K) {
      while (v >= vcnt) {
        if (hops == 7) return -1;
        ++hops;
        vx = (vx + 1) & 7;
        vbeg = bound(vx);
        vcnt = bound(vx + 1) - vbeg;
        lds_barrier();  // every wave has read the mailbox
        if (tid == 0) *mbox = atomicAdd(args.queue + vx, 1);
        lds_barrier();
        v = __builtin_amdgcn_readfirstlane(*mbox);
      }
      return vbeg + v;
    } else {
      return v;
    }
  };
  auto done = [&](int t) { return Tr::GROUP_K ? t < 0 : t >= total; };
  auto coord = [&](int tile) -> TileCoord {
    TileCoord c{};
    if constexpr (!Tr::GROUP_K) {
      // (expert, n-tile, m-tile) order; expert e owns tiles [tp[e]*ntn, tp[e+1]*ntn),
      // so e is the last expert with tp[e] <= tile / ntn
      const int q = tile / ntn;
      int lo = 0, hi = E_loc - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sload(tp + mid) <= q) lo = mid; else hi = mid - 1;
      }
      c.e_loc = lo;
      const int t0 = sload(tp + lo), t1 = sload(tp + lo + 1);
      int mt, nt;
      tile_mn<MOK_ROW_GM>(tile - t0 * ntn, t1 - t0, ntn, mt, nt);
      c.n0 = nt * BN;
      const int e = args.eb + lo;
      c.row0 = sload(args.offsets + e) + mt * BM;
      c.row_end = sload(args.offsets + e + 1);
    } else {
      const int per_z = ntm_k * ntn;
      const int g = tile;  // position in the heaviest-first sequence
      const i32x4_t rec = sload4(args.expert_order + 4 * (g / (NZ * per_z)));
      c.e_loc = rec[0];
      c.row0 = rec[1];
      c.row_end = rec[2];
      const int rem = g % (NZ * per_z);
      c.z = rem / per_z;
      int mt, nt;
      tile_mn<2>(rem % per_z, ntm_k, ntn, mt, nt);
      c.m0 = mt * BM;
      c.n0 = nt * BN;
    }
    return uniform(c);
  };

  int tile = vb;
  if constexpr (Tr::GROUP_K) {
    take();
    if (tid == 0) *mbox = taken;
    lds_barrier();
    tile = resolve(__builtin_amdgcn_readfirstlane(*mbox));
    lds_barrier();
  }
  if (done(tile)) return;
  Job cur;
  cur.init(args, coord(tile));
  cur.prologue(arena);
  f32x16_t acc[Job::NB][Job::FM][Job::FN];
  while (true) {
    take();
    cur.mainloop(acc, arena);
    int nt = tile + G_;
    if constexpr (Tr::GROUP_K) {
      if (tid == 0) *mbox = taken;
    }
    lds_barrier();  // every wave is done with the stage buffers (and sees the mailbox)
    if constexpr (Tr::GROUP_K) nt = resolve(__builtin_amdgcn_readfirstlane(*mbox));
    typename Job::SavedAB pre;
    cur.epilogue_prefetch(pre);
    Job nxt = cur;
    if (!done(nt)) {
      nxt.init(args, coord(nt));
      nxt.prologue(arena);
    }
    // the next mailbox write follows a barrier of the next K loop, which
    // has one whenever it has a stage
    if (Tr::GROUP_K && (done(nt) || nxt.nk == 0)) lds_barrier();
    cur.epilogue(acc, staging, pre);
    if (done(nt)) break;
    cur = nxt;
    tile = nt;
  }
#endif
}

template <int KIND, int BM, int BN, int NS, int BK, int NW, int WMW>
static hipError_t run_bf16(const GroupedGemmArgs& g, hipStream_t s) {
  const GemmGeom G = geom_of<KIND>(g.d, g.F);
  const int ntn = (G.N + BN - 1) / BN;
  int blocks;
  if constexpr (Traits<KIND>::GROUP_K) {
    // persistent workers over the 8 per-XCD tile counters (zeroed earlier on
    // the stream); a multiple of 8 workgroups so that every counter is served
    blocks = 256;
  } else {
    // persistent: one workgroup per CU, bounded by the worst-case tile count
    const int64_t worst = ((g.P_max + BM - 1) / BM + g.E_loc) * (int64_t)ntn;
    blocks = (int)(worst < 256 ? worst : 256);
  }
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<KIND, BM, BN, NS, BK, NW, WMW>), dim3(blocks), dim3(NW * 64), 0, s,
                     g);
  return hipGetLastError();
}

// Stage depth (BK) and count (NS) per kind: 32 x 4 or 64 x 2 fill the LDS.
// DH and DX take two 64-K stages: their K-contiguous A rows are then whole
// 128-byte pieces, which the copy path serves about twice as fast as 64-byte
// ones (same-box A/B at T 8192, d 4096, E 128, k 8, F 1536: DH 1.32 -> 1.23
// ms, DX 2.19 -> 2.01 ms).
// UP and DOWN (eight waves) take two 64-K stages too, with 16-row epilogue
// rounds (4 KB of staging per wave): same-box A/B UP 1.94 -> 1.86 ms, DOWN
// 1.03 -> 0.99 ms against three 32-K stages.
#ifndef MOK_UPDN_BK64
#define MOK_UPDN_BK64 1
#endif
#ifndef MOK_BK_UP
#define MOK_BK_UP (MOK_UPDN_BK64 ? 64 : 32)
#define MOK_BK_DOWN (MOK_UPDN_BK64 ? 64 : 32)
#define MOK_NS_DH 2
#define MOK_BK_DH 64
#define MOK_NS_DX 2
#define MOK_BK_DX 64
#define MOK_NS_DW 4
#define MOK_BK_DW 32
#endif
// dW2 takes 64-K stages, two of them (same-box A/B: 1.43 -> 1.40 ms); dW1/dW3
// keeps 32 x 4 (64 x 2: 2.74 -> 2.83 ms).
#ifndef MOK_BK_DW2
#define MOK_NS_DW2 2
#define MOK_BK_DW2 64
#endif

// Waves per workgroup and their layout per kind.  UP and DOWN (both operands
// K-contiguous) run eight waves, 4 x 2, with three stage buffers (their
// staging then takes 64 KB of the LDS): 2.05 -> 1.90 ms and 1.14 -> 1.05 ms
// at T 8192, d 4096, E 128, k 8, F 1536.  DH and DX measured slower with
// eight waves in either layout (DH 1.30 -> 1.44-1.51 ms, DX 2.19 -> 2.34-
// 2.40) with 32-K stages.
#ifndef MOK_BF16_WAVES_FWD
#define MOK_BF16_WAVES_FWD 8
#endif
constexpr int kWF = MOK_BF16_WAVES_FWD;
// dW2 runs eight waves, 2 x 4 (same-box A/B: 1.44 -> 1.34-1.38 ms); dW1/dW3
// keeps four (eight, 2 x 4 or 4 x 2: 2.68-2.73 -> 2.80-2.84 ms).
#ifndef MOK_BF16_WAVES_DW
#define MOK_BF16_WAVES_DW 8
#endif
#ifndef MOK_BF16_WM_DW
#define MOK_BF16_WM_DW 2
#endif
constexpr int kWDW = MOK_BF16_WAVES_DW, kWmDW = MOK_BF16_WM_DW;
// DX with 64-K stages runs eight waves, 2 x 4 (its transposing B reads then
// serve two waves per fragment; 16-row epilogue rounds): same-box A/B 2.00 ->
// 1.82 ms (4 x 2: 1.84 ms).  DH keeps four (its epilogue prefetches whole
// 32-row rounds of the saved A and B).
#ifndef MOK_DX_WAVES
#define MOK_DX_WAVES 8
#define MOK_DX_WM 2
#endif
constexpr int kNsFwd = MOK_UPDN_BK64 ? 2 : (kWF == 8 ? 3 : 4);

hipError_t gemm_bf16(int kind, const GroupedGemmArgs& g, hipStream_t s) {
  switch (kind) {
    case KIND_UP:   return run_bf16<KIND_UP, 256, 128, kNsFwd, MOK_BK_UP, kWF, kWF / 2>(g, s);
    case KIND_DOWN: return run_bf16<KIND_DOWN, 256, 256, kNsFwd, MOK_BK_DOWN, kWF, kWF / 2>(g, s);
    case KIND_DH:   return run_bf16<KIND_DH, 256, 256, MOK_NS_DH, MOK_BK_DH, 4, 2>(g, s);
    case KIND_DX:   return run_bf16<KIND_DX, 256, 256, MOK_NS_DX, MOK_BK_DX, MOK_DX_WAVES, MOK_DX_WM>(g, s);
    case KIND_DW2:  return run_bf16<KIND_DW2, 256, 256, MOK_NS_DW2, MOK_BK_DW2, kWDW, kWmDW>(g, s);
    case KIND_DW13: return run_bf16<KIND_DW13, 256, 256, MOK_NS_DW, MOK_BK_DW, 4, 2>(g, s);
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
__device__ __forceinline__ TileCoord range_tile(const GroupedGemmArgs& g, const int32_t* s_tp, int ntn, int BM,
                                                int r0, int r1, int t, int BN) {
  int lo = 0, hi = g.E_loc - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_tp[mid] * ntn <= t) lo = mid; else hi = mid - 1;
  }
  TileCoord c{};
  c.e_loc = lo;
  const int mt_e = s_tp[lo + 1] - s_tp[lo];
  const int local = t - s_tp[lo] * ntn;
  c.n0 = (local / mt_e) * BN;
  c.row0 = max(g.offsets[g.eb + lo], r0) + (local % mt_e) * BM;
  c.row_end = min(g.offsets[g.eb + lo + 1], r1);
  return uniform(c);
}

// A whole tile with no overlap between tiles (issue, K loop, epilogue), with
// four stage buffers in an arena of kRingArena bytes (the ring kernel keeps
// its range tables in LDS too).  The epilogue staging (8 KB per wave) sits
// behind the stage buffers where they leave room, else in the last stage
// buffer, free once the K loop is done.
constexpr int kRingStages = 4;
constexpr int kRingArena = 128 * 1024;
template <int KIND, int BM, int BN>
__device__ __forceinline__ void run_tile(const GroupedGemmArgs& g, const TileCoord& c, uint8_t* arena) {
  using Job = TileJob<KIND, BM, BN, kRingStages, 32>;
  constexpr int kStaging = 4 * Job::EP_BYTES;
  constexpr bool kBehind = kRingStages * Job::STAGE + kStaging <= kRingArena;
  static_assert(kRingStages * Job::STAGE <= kRingArena && (kBehind || Job::STAGE >= kStaging), "ring arena");
  Job job;
  job.init(g, c);
  job.prologue(arena);
  f32x16_t acc[Job::NB][Job::FM][Job::FN];
  job.mainloop(acc, arena);
  lds_barrier();
  typename Job::SavedAB pre;
  job.epilogue_prefetch(pre);
  job.epilogue(acc, arena + (kBehind ? kRingStages : kRingStages - 1) * Job::STAGE, pre);
  lds_barrier();
}

// Row tiles of the ring kernel's two GEMMs: UP tiles of 128 rows (128 F
// columns of both W1 and W3 over K = d) and DOWN tiles of 256 rows (256
// columns over K = F), so that a minibatch of R rows makes about twice as
// many UP tiles as 256-row tiles would, each half as long: a launch lasts
// about as long as its longest tile.  Each output element is still the same
// MFMA sequence over K as in the whole-layer GEMMs.
#ifndef MOK_RING_BM_UP
#define MOK_RING_BM_UP 128
#endif
#ifndef MOK_RING_BM_DOWN
#define MOK_RING_BM_DOWN 256
#endif
// 16-byte loads each lane of a copy task issues before their stores.
#ifndef MOK_RING_COPY_UNROLL
#define MOK_RING_COPY_UNROLL 8
#endif

[[maybe_unused]] constexpr int kCopyRows = 16;  // rows per copy task

// Copy task t: rows [c0 + 16 t, ...) of the next minibatch (at most c1) from
// their tokens' rows of x into the ring slot, MOK_RING_COPY_UNROLL 16-byte
// loads per lane issued before their stores.
__device__ __forceinline__ void copy_task(const MinibatchStepArgs& a, int t, int c0, int c1) {
  constexpr int CU = MOK_RING_COPY_UNROLL;
  const int tid = threadIdx.x, d = a.up.d, nv = d / 8;
  const int rb = c0 + t * kCopyRows, re = min(rb + kCopyRows, c1);
  const int n = (re - rb) * nv;
  for (int v0 = tid; v0 < n; v0 += 256 * CU) {
    u32x4_t val[CU];
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const int v = v0 + u * 256;
      if (v < n) {
        const int tok = a.pair_of_row[rb + v / nv] / a.k;
        val[u] = reinterpret_cast<const u32x4_t*>((const bf16_t*)a.x + (int64_t)tok * d)[v % nv];
      }
    }
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const int v = v0 + u * 256;
      if (v < n) reinterpret_cast<u32x4_t*>((bf16_t*)a.ring_dst + (int64_t)(rb + v / nv - c0) * d)[v % nv] = val[u];
    }
  }
}

__global__ __launch_bounds__(256) void minibatch_step_kernel(MinibatchStepArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BMU = MOK_RING_BM_UP, BMD = MOK_RING_BM_DOWN;
  __shared__ __attribute__((aligned(1024))) uint8_t arena[kRingArena];
  __shared__ int32_t s_up[1025], s_dn[1025], s_wsum[4];
  const int tid = threadIdx.x;
  const GroupedGemmArgs& gu = a.up;
  const int P = gu.offsets[gu.eb + gu.E_loc];  // local rows
  const int u0 = min(a.up0, P), u1 = min(a.up1, P);
  const int d0 = min(a.dn0, P), d1 = min(a.dn1, P);
  const int c0 = min(a.cp0, P), c1 = min(a.cp1, P);
  range_tile_prefix<BMU>(gu, u0, u1, s_up, s_wsum);
  range_tile_prefix<BMD>(a.down, d0, d1, s_dn, s_wsum);
  const int ntn_up = (gu.F + 127) / 128, ntn_dn = (gu.d + 255) / 256;
  const int n_cp = (c1 - c0 + kCopyRows - 1) / kCopyRows;
  const int n_up = s_up[gu.E_loc] * ntn_up;
  const int n_dn = s_dn[gu.E_loc] * ntn_dn;
  const int G_ = gridDim.x;
  const int movers = a.movers > 0 && a.movers < G_ ? a.movers : 0;
  // Tasks: n_cp row copies, n_up UP tiles, n_dn DOWN tiles.  With movers,
  // workgroups b < movers (spread over the XCDs, b % 8) take the copies b,
  // b + movers, ... and the other workgroups only the tiles.  The tiles (and,
  // without movers, the copies) are cut into eight runs: run x holds the x-th
  // eighth of the UP tiles, then of the DOWN tiles, then of the copies, so
  // the longest tasks of a run come first and neighbouring tiles, which read
  // the same weight columns, share an XCD's L2.  The workgroups of XCD x take
  // run x's tasks in order from counter x and, once it is exhausted, those of
  // the next runs in turn; which workgroup runs a task never changes what it
  // computes.  The last workgroup to finish leaves every counter at zero for
  // the next launch.
  const int n_rcp = movers ? 0 : n_cp;
  auto cut = [](int n, int x) { return (int)(((int64_t)n * x) >> 3); };
  auto run_len = [&](int x) {
    return cut(n_up, x + 1) - cut(n_up, x) + cut(n_dn, x + 1) - cut(n_dn, x) + cut(n_rcp, x + 1) - cut(n_rcp, x);
  };
  // Task index (copies first, then UP, then DOWN) of position v of run x.
  auto run_task = [&](int x, int v) {
    const int lu = cut(n_up, x + 1) - cut(n_up, x);
    if (v < lu) return n_cp + cut(n_up, x) + v;
    v -= lu;
    const int ld = cut(n_dn, x + 1) - cut(n_dn, x);
    if (v < ld) return n_cp + n_up + cut(n_dn, x) + v;
    return cut(n_rcp, x) + v - ld;
  };
  __shared__ int s_take;
  auto take = [&](int x) -> int {
    if (tid == 0) s_take = atomicAdd(a.ctr + x, 1);
    __syncthreads();
    const int v = __builtin_amdgcn_readfirstlane(s_take);
    __syncthreads();
    return v;
  };
  if ((int)blockIdx.x < movers) {
    for (int t = blockIdx.x; t < n_cp; t += movers) copy_task(a, t, c0, c1);
  } else {
    int x = blockIdx.x % 8;
    for (int hop = 0; hop < 8; ++hop, x = (x + 1) & 7) {
      const int len = run_len(x);
      for (int v = take(x); v < len; v = take(x)) {
        const int t = run_task(x, v);
        if (t < n_cp) {
          copy_task(a, t, c0, c1);
        } else if (t < n_cp + n_up) {
          run_tile<KIND_UP, BMU, 128>(gu, range_tile(gu, s_up, ntn_up, BMU, u0, u1, t - n_cp, 128), arena);
        } else {
          run_tile<KIND_DOWN, BMD, 256>(a.down, range_tile(a.down, s_dn, ntn_dn, BMD, d0, d1, t - n_cp - n_up, 256),
                                        arena);
        }
      }
    }
  }
  if (tid == 0) {
    // every workgroup has taken its last task index once this count is full
    if (atomicAdd(a.ctr + 8, 1) == G_ - 1)
      for (int i = 0; i < kRingCounters; ++i) atomicExch(a.ctr + i, 0);
  }
#endif
}

hipError_t launch_minibatch_step(const MinibatchStepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(minibatch_step_kernel, dim3(256), dim3(256), 0, s, a);
  return hipGetLastError();
}

__global__ void ring_reset_kernel(int32_t* ctr) {
  if (threadIdx.x < kRingCounters) ctr[threadIdx.x] = 0;
}

hipError_t launch_ring_reset(int32_t* ctr, hipStream_t s) {
  hipLaunchKernelGGL(ring_reset_kernel, dim3(1), dim3(64), 0, s, ctr);
  return hipGetLastError();
}

}  // namespace mok
