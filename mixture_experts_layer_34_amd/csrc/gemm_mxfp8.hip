// Expert-grouped MXFP8 GEMMs (gfx950 v_mfma_scale_f32_32x32x64_f8f6f4):
//   UP    H_e = silu(X_e W1_e^T) * (X_e W3_e^T), quantised to MXFP8 along F
//   DOWN  Y_e = H_e W2_e^T (bf16)
// and the backward products that flow on to dx, each operand quantised along
// the axis it contracts (the weights as transposed copies, see
// mok_quantize_mxfp8_backward_weights):
//   DH    dH_e = dY_e (W2_e^T)^T, then the SwiGLU backward: dA, dB (bf16, for
//         the weight gradients) and [dA | dB] quantised along F
//   DX    dX_e = [dA | dB]_e [W1_e^T | W3_e^T]^T (bf16), K = 2F
// and the weight gradients, whose contraction runs over the expert's rows:
//   DW2   dW2_e = Qr(dY_e)^T Qr(H_e)                 (fp32 [d, F])
//   DW13  [dW1_e; dW3_e] = Qr([dA | dB]_e)^T Qr(X_e) (fp32 [F, d] each)
// with the operands quantised along the rows and stored transposed, so that
// they too are K-contiguous (see quantize_rows.hip): A row m is column m of
// the row-major operand, K runs over the expert's padded row segment.
// Operands are E4M3 with one E8M0 scale per 32 consecutive K values (OCP MX
// v1.0).  MXFP8 activation quantisation sits in the dispatch, grouped-GEMM and
// SwiGLU data paths instead of a standalone kernel (kucoin.com, "Cursor's MoK
// réalise une amélioration des performances de 2,37x sur NVIDIA GB300 NVL72",
// section 02): X rows are quantised by the dispatch gather, H by this UP
// epilogue, and the scaled MFMA consumes both without dequantising.
//
// The pipeline is the bf16 one (gemm_bf16.hip) with one-byte elements: a
// stage is 128 K values = two scaled-MFMA K steps = 128-byte LDS rows, two
// stage buffers, the same swizzle, direct-to-LDS copies, barrier placement
// and tile schedule.  The copy path serves whole 128-byte row pieces about
// twice as fast as 64-byte ones: against 64-K stages (four buffers) at T
// 8192, d 4096, E 128, k 8, F 1536, UP 1.69 -> 1.59 ms, DOWN 0.90 -> 0.82,
// DH 1.07 -> 1.03, DX 1.60 -> 1.45 (same-box A/B).  Each stage also carries
// the two E8M0 bytes of every tile row for each of its K steps (2-byte
// copies that land zero-extended in one LDS dword per row).  Scales are
// stored in pair planes (see mok_quantize_mxfp8): the two bytes of one row
// for one K step are a 2-byte word of plane k / 64, next to those of the
// next row, so a wave's scale copy reads 128 contiguous bytes.
// Scaled-MFMA operand layout on gfx950 (checked on the device): lane l holds
// row l % 32; with h = l / 32 its bytes 0-15 are K [16h, 16h + 16) and bytes
// 16-31 are K [32 + 16h, +16), and the scale it supplies covers the 32-block
// h of the step — byte h of the row's scale dword, shifted down to byte 0.
#include "mok_device.h"
#include "mok_internal.h"
#include "gemm_common.h"
#include "gemm_pipe.h"

namespace mok {

constexpr int kMxNS = 5;     // LDS stage buffers (4-wave workgroups)
// Row tiles: skip the MFMAs of 32-row blocks wholly past the expert's end.
#ifndef MOK_SKIP_PAD
#define MOK_SKIP_PAD 1
#endif
#ifndef MOK_MX_GM
#define MOK_MX_GM 4  // m-tiles per raster group (tile_mn)
#endif
#ifndef MOK_MX_WAVES
#define MOK_MX_WAVES 8
#endif
// Weight-gradient kinds: non-temporal fp32 stores, so that the dW lines do
// not take L2 space from the operands (same-box A/B at T 8192, d 4096, E 128,
// k 8, F 1536: dW1/dW3 2.69 -> 2.50 ms, dW2 1.32 -> 1.27 ms).  Measured and
// dropped: dealing whole experts to the XCDs (snake order of their rank,
// row-tile-major tiles on each XCD's own workgroups, so that an expert's
// operands are fetched into one L2 only): 3.43 and 1.60 ms.
#ifndef MOK_MXW_NT_STORE
#define MOK_MXW_NT_STORE 1
#endif
constexpr int kMxWaves = MOK_MX_WAVES;

__device__ __forceinline__ u32x4_t pack_bf16x8(const float* v) {
  u32x4_t w;
#pragma unroll
  for (int t = 0; t < 4; ++t) w[t] = (uint32_t)f2bf(v[2 * t]) | ((uint32_t)f2bf(v[2 * t + 1]) << 16);
  return w;
}
// E4M3 codes of v[0..7] / 2^se
__device__ __forceinline__ u32x2_t pack_e4m3x8(const float* v, int se) {
  u32x2_t w;
  w[0] = e4m3x4(ldexpf(v[0], -se), ldexpf(v[1], -se), ldexpf(v[2], -se), ldexpf(v[3], -se));
  w[1] = e4m3x4(ldexpf(v[4], -se), ldexpf(v[5], -se), ldexpf(v[6], -se), ldexpf(v[7], -se));
  return w;
}
#ifndef MOK_MX_BK
#define MOK_MX_BK 128
#endif
constexpr int kMxBK = MOK_MX_BK;    // bytes of K per stage (E4M3: one (64) or two (128) MFMA K steps)
constexpr int kMxLPR = kMxBK / 16;  // lanes per row in a 1 KB copy
// Operand formats, as the scaled MFMA encodes them.  E2M1 (MXFP4) operands
// hold two codes per byte, so a stage of kMxBK bytes holds twice the K
// values, and an MFMA K step (64 values) is 32 bytes: a lane (row l % 32,
// h = l / 32) then holds the 16 bytes [16 h, 16 h + 16) of the step, K values
// [32 h, 32 h + 32), the lower one in the low nibble (checked on the device).
constexpr int kFmtE4M3 = 0, kFmtE2M1 = 4;

// One MXFP8 output tile (UP: 256 rows x 64 columns of W1 and W3; DOWN:
// 256 x 128): 128 accumulators per lane, which leaves the register file room
// for the fragments (at one byte per element this tile moves the same L2
// bytes per FLOP as the 256 x 256 bf16 tile).  Wave-uniform members except
// the per-lane DMA offsets.
// Contraction length and output columns of each kind.
template <int KIND> __host__ __device__ inline int mx_k(int d, int F) {
  return KIND == KIND_UP || KIND == KIND_DH ? d : (KIND == KIND_DX ? 2 * F : F);
}
template <int KIND> __host__ __device__ inline int mx_n(int d, int F) {
  return KIND == KIND_UP || KIND == KIND_DH || KIND == KIND_DW2 ? F : d;
}
// Weight-gradient kinds: output rows (dW2: d; DW13: dW1 rows then dW3 rows).
template <int KIND> __host__ __device__ inline int mx_m(int d, int F) { return KIND == KIND_DW2 ? d : 2 * F; }
template <int KIND> constexpr bool mx_wgrad() { return KIND == KIND_DW2 || KIND == KIND_DW13; }

// NW waves per workgroup: NW = 4 as 2 x 2 waves of 128 x TN (128
// accumulators); NW = 8 as 4 x 2 waves of 64 x TN (64 accumulators, two waves
// per SIMD, so that one wave's MFMAs can run while the other waits to issue
// its copies).
template <int KIND, int NW, int FMT = kFmtE4M3>
struct MxJob {
  static constexpr int EPB = FMT == kFmtE2M1 ? 2 : 1;  // K values per byte
  static constexpr int SUB = kMxBK * EPB / 64;         // MFMA K steps per stage
  static constexpr int KST = kMxBK * EPB;              // K values per stage
  static_assert(FMT == kFmtE4M3 || (KIND == KIND_UP || KIND == KIND_DOWN), "E2M1: forward kinds only");
  static constexpr int NB = KIND == KIND_UP ? 2 : 1;
  static constexpr int BM = 256, BN = KIND == KIND_UP ? 64 : 128, BROWS = NB * BN;
  static constexpr int WM = NW / 2;                   // waves along M (2 along N)
  static constexpr int TM = BM / WM, TN = BN / 2, FM = TM / 32, FN = TN / 32;
  static constexpr int NS = NW == 4 ? kMxNS : (SUB == 1 ? 4 : 2);  // LDS stage buffers
  static constexpr int A_BYTES = BM * kMxBK, B_BYTES = BROWS * kMxBK;
  // Scale dwords (each 2-byte copy lands zero-extended in one dword); every
  // wave issues one A-scale and one B-scale copy of RA resp. RB rows, whose
  // lanes past those rows read outside the resource into unused dwords:
  //   A row r at dword 64 (r / RA) + r % RA, B row r at dword 64 (r / RB) + r % RB.
  static constexpr int RA = BM / NW, RB = BROWS / NW;
  static constexpr int SCA = A_BYTES + B_BYTES;
  static constexpr int SCB = SCA + SUB * NW * 256;   // (one scale set per MFMA K step)
  static constexpr int STAGE = SCB + SUB * NW * 256;
  static constexpr int IA = A_BYTES / 1024 / NW, IB = B_BYTES / 1024 / NW;  // 1 KB copies per wave
  static constexpr int D = IA + IB + 2 * SUB;         // + one 2-byte copy per wave for each scale set
  static constexpr int STAGING = NW * 4096;           // epilogue staging, 4 KB per wave
  static_assert(BM == 256 && BROWS == 128 && FM % 2 == 0, "tile");
  static_assert((NS - 1) * D <= 63, "vmcnt holds at most 63");
  static_assert(NS * STAGE + STAGING <= 163840, "LDS");

  struct AFrag {  // one 32-row block of A for one K step, with its scales
    i32x8_t v;
    uint32_t s;
  };
  struct BFrags {  // all B blocks of a wave for one K step
    i32x8_t v[NB][FN];
    uint32_t s[NB][FN];
  };

  const GroupedGemmArgs* args;
  int K, N;
  uint32_t lda, ldb;  // bytes per operand row (K / EPB for the row kinds, k_pad for the weight gradients)
  uint32_t psA, psB;  // bytes per scale plane of A (P_max rows) and of B (E_loc * N rows)
  TileCoord c;
  int wid, lane, wm, wn, nk;
  int nvb;  // this wave's 32-row blocks that hold rows of the expert (the rest: no MFMAs)
  i32x4_t rsA, rsB0, rsB1, rsSA, rsSB0, rsSB1;
  uint32_t offA[IA], offB[IB], offSA, offSB;

  __device__ __forceinline__ void init(const GroupedGemmArgs& a, const TileCoord& tc) {
    args = &a;
    N = mx_n<KIND>(a.d, a.F);
    c = tc;
    lane = threadIdx.x & 63;
    wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    wm = wid >> 1;
    wn = wid & 1;
    nvb = FM;
    if constexpr (mx_wgrad<KIND>()) {
      init_wgrad(a);
      return;
    }
    K = mx_k<KIND>(a.d, a.F);
    const int Kb = K / EPB;  // bytes per operand row
    lda = ldb = (uint32_t)Kb;
    nk = K / KST;
    if (MOK_SKIP_PAD) {
      // rows past the expert's end are zero padding and are never stored:
      // their MFMAs are skipped (less work, less power)
      const int left = c.row_end - (c.row0 + wm * TM);
      nvb = left <= 0 ? 0 : (left >= TM ? FM : (left + 31) / 32);
    }
    const int rows = c.row_end - c.row0 < BM ? c.row_end - c.row0 : BM;
    const int nb_rows = N - c.n0 < BN ? N - c.n0 : BN;
    const int64_t wst = (int64_t)N * Kb;  // bytes per expert of one weight matrix
    rsA = make_rsrc((const uint8_t*)a.A + (int64_t)c.row0 * Kb, (uint32_t)(rows * Kb));
    rsB0 = make_rsrc((const uint8_t*)a.B0 + c.e_loc * wst + (int64_t)c.n0 * Kb, (uint32_t)(nb_rows * Kb));
    rsB1 = make_rsrc((const uint8_t*)(NB == 2 ? a.B1 : a.B0) + c.e_loc * wst + (int64_t)c.n0 * Kb,
                     (uint32_t)(nb_rows * Kb));
    // scale resources from this tile's first row to the end of the last
    // plane; rows past the tile read other rows' bytes (finite E8M0 codes, or
    // zero past the end), which only reach output rows that are not stored
    const int64_t pa = (int64_t)a.P_max * 2, pb = (int64_t)a.E_loc * N * 2;
    psA = (uint32_t)pa;
    psB = (uint32_t)pb;
    const int64_t planes = K / 64;
    const int64_t fb = ((int64_t)c.e_loc * N + c.n0) * 2;
    rsSA = make_rsrc(a.a_scale + (int64_t)c.row0 * 2, (uint32_t)(planes * pa - (int64_t)c.row0 * 2));
    rsSB0 = make_rsrc(a.b_scale0 + fb, (uint32_t)(planes * pb - fb));
    rsSB1 = make_rsrc((NB == 2 ? a.b_scale1 : a.b_scale0) + fb, (uint32_t)(planes * pb - fb));
    init_offsets();
  }

  // Weight-gradient tile: rows m0 .. m0 + 255 of the output (columns of the
  // row-major A operand), columns n0 .. n0 + 127, K over the expert's padded
  // segment [row0, row_end) of the transposed operands (row stride k_pad
  // bytes; scale planes of M_total resp. N rows).  Every output row is real:
  // no row blocks are skipped; an expert without rows has nk = 0 and stores
  // zeros.
  __device__ __forceinline__ void init_wgrad(const GroupedGemmArgs& a) {
    const int M = mx_m<KIND>(a.d, a.F);
    const int kbeg = c.row0;
    K = c.row_end - c.row0;
    nk = K / kMxBK;
    lda = ldb = (uint32_t)a.k_pad;
    rsA = make_rsrc((const uint8_t*)a.A + (int64_t)c.m0 * a.k_pad + kbeg, (uint32_t)(BM * a.k_pad - kbeg));
    rsB0 = make_rsrc((const uint8_t*)a.B0 + (int64_t)c.n0 * a.k_pad + kbeg, (uint32_t)(BN * a.k_pad - kbeg));
    rsB1 = rsB0;
    psA = (uint32_t)(M * 2);
    psB = (uint32_t)(N * 2);
    const int64_t p0 = kbeg / 64, planes = K / 64;
    rsSA = make_rsrc(a.a_scale + p0 * psA + (int64_t)c.m0 * 2, (uint32_t)(planes * psA - (int64_t)c.m0 * 2));
    rsSB0 = make_rsrc(a.b_scale0 + p0 * psB + (int64_t)c.n0 * 2, (uint32_t)(planes * psB - (int64_t)c.n0 * 2));
    rsSB1 = rsSB0;
    init_offsets();
  }

  __device__ __forceinline__ void init_offsets() {
#pragma unroll
    for (int q = 0; q < IA; ++q) {
      const int r = (wid * IA + q) * (64 / kMxLPR) + lane / kMxLPR;
      offA[q] = (uint32_t)(r * lda + swz_k<kMxBK / 2>(r, lane % kMxLPR) * 16);
    }
#pragma unroll
    for (int q = 0; q < IB; ++q) {
      const int r = (wid * IB + q) * (64 / kMxLPR) + lane / kMxLPR;
      const int rl = (NB == 2 && r >= BN) ? r - BN : r;
      offB[q] = (uint32_t)(rl * ldb + swz_k<kMxBK / 2>(r, lane % kMxLPR) * 16);
    }
    // scale copies: wave w brings A rows 64 w .. 64 w + 63 and, in lanes 0-31,
    // B rows 32 w .. 32 w + 31 (UP: of W1 for w < 2, of W3 after); lanes 32-63
    // of the B copy read past the resource and land zero in unused dwords
    offSA = lane < RA ? (uint32_t)((wid * RA + lane) * 2) : 0xFFFFFFF0u;
    const int rb = wid * RB + lane;
    offSB = lane < RB ? (uint32_t)(((NB == 2 && rb >= BN) ? rb - BN : rb) * 2) : 0xFFFFFFF0u;
  }

  // Copies [Q0, Q1) of stage s (A data, B data, A scales, B scales).
  template <int Q0, int Q1>
  __device__ __forceinline__ void issue_part(int s, uint8_t* arena) const {
    uint8_t* st = arena + (s % NS) * STAGE;
    const int k0 = s * kMxBK;
#pragma unroll
    for (int q = 0; q < IA; ++q)
      if (q >= Q0 && q < Q1) dma_b128(rsA, lds_addr(st + (wid * IA + q) * 1024), offA[q], k0);
#pragma unroll
    for (int q = 0; q < IB; ++q)
      if (IA + q >= Q0 && IA + q < Q1)
        dma_b128((NB == 2 && (wid * IB + q) * (64 / kMxLPR) >= BN) ? rsB1 : rsB0,
                 lds_addr(st + A_BYTES + (wid * IB + q) * 1024), offB[q], k0);
#pragma unroll
    for (int p = 0; p < SUB; ++p) {  // scale plane s * SUB + p
      const uint32_t plane = (uint32_t)(s * SUB + p);
      if (IA + IB + 2 * p >= Q0 && IA + IB + 2 * p < Q1)
        dma_u16(rsSA, lds_addr(st + SCA + (p * NW + wid) * 256), offSA, plane * psA);
      if (IA + IB + 2 * p + 1 >= Q0 && IA + IB + 2 * p + 1 < Q1)
        dma_u16((NB == 2 && wid * RB >= BN) ? rsSB1 : rsSB0, lds_addr(st + SCB + (p * NW + wid) * 256), offSB,
                plane * psB);
    }
  }
  __device__ __forceinline__ void issue(int s, uint8_t* arena) const { issue_part<0, D>(s, arena); }

  // One operand row's fragment for MFMA K step `sub` of a stage (h = lane /
  // 32): E4M3, the 16-byte chunks 4 sub + h and 4 sub + 2 + h of the row;
  // E2M1, the chunk 2 sub + h (the upper half of the operand is not read).
  __device__ __forceinline__ static i32x8_t frag(const uint8_t* row, int r, int sub, int h) {
    if constexpr (FMT == kFmtE2M1) {
      const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(row + swz_k<kMxBK / 2>(r, 2 * sub + h) * 16);
      const i32x4_t z = {0, 0, 0, 0};
      return __builtin_shufflevector(lo, z, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
      const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(row + swz_k<kMxBK / 2>(r, 4 * sub + h) * 16);
      const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(row + swz_k<kMxBK / 2>(r, 4 * sub + 2 + h) * 16);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
  // Fragments of MFMA K step `sub` of a stage, and that step's scale set.
  __device__ __forceinline__ void read_a(int buf, int i, int sub, const uint8_t* arena, AFrag& f) const {
    const uint8_t* st = arena + buf * STAGE;
    const int h = lane >> 5;
    const int r = wm * TM + i * 32 + (lane & 31);
    f.v = frag(st + r * kMxBK, r, sub, h);
    f.s = *reinterpret_cast<const uint32_t*>(st + SCA + sub * NW * 256 + (64 * (r / RA) + r % RA) * 4) >> (8 * h);
  }
  __device__ __forceinline__ void read_b(int buf, int sub, const uint8_t* arena, BFrags& f) const {
    const uint8_t* st = arena + buf * STAGE;
    const int h = lane >> 5;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = b * BN + wn * TN + j * 32 + (lane & 31);
        f.v[b][j] = frag(st + A_BYTES + r * kMxBK, r, sub, h);
        f.s[b][j] =
            *reinterpret_cast<const uint32_t*>(st + SCB + sub * NW * 256 + (64 * (r / RB) + r % RB) * 4) >> (8 * h);
      }
  }

  // MFMAs of row block i (all B blocks), [g, g + 1) / NG of them.
  template <int g, int NG>
  __device__ __forceinline__ void mma_row(f32x16_t (&acc)[NB][FM][FN], int i, const AFrag& fa,
                                          const BFrags& fb) const {
    if (i >= nvb) return;
    constexpr int TOT = NB * FN, L0 = g * TOT / NG, L1 = (g + 1) * TOT / NG;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int L = b * FN + j;
        if (L >= L0 && L < L1)
          acc[b][i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa.v, fb.v[b][j], acc[b][i][j], FMT, FMT,
                                                                          0, (int)fa.s, 0, (int)fb.s[b][j]);
      }
  }

  // Last row block's MFMAs with stage s's copies spread between them.
  template <int G, int NG>
  __device__ __forceinline__ void mma_issue(f32x16_t (&acc)[NB][FM][FN], const AFrag& fa, const BFrags& fb,
                                            bool copy, int s, uint8_t* arena) const {
    if constexpr (G < NG) {
      if (copy) issue_part<G * D / NG, (G + 1) * D / NG>(s, arena);
      __builtin_amdgcn_sched_barrier(0);
      mma_row<G, NG>(acc, FM - 1, fa, fb);
      __builtin_amdgcn_sched_barrier(0);
      mma_issue<G + 1, NG>(acc, fa, fb, copy, s, arena);
    }
  }

  // K loop, one MFMA K step per stage.  A stage's B blocks are read during the
  // previous stage; its A row blocks are read one block ahead of the MFMAs
  // that use them.  Once a wave has read the stage's last A block, it waits
  // for the next stage and meets the workgroup (every wave is then done with
  // this stage's buffer), reads the next stage's B blocks and first A block,
  // and runs the last row block's MFMAs with the copies of stage kt + NS
  // spread between them.  On entry stages 0 .. min(nk, NS) - 1 are issued.
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
    wait_stages<D, NS - 1>(nk - 1 < NS - 1 ? nk - 1 : NS - 1);
    BFrags b0, b1;
    AFrag a0, a1;
    read_b(0, 0, arena, b0);
    read_a(0, 0, 0, arena, a0);
    if constexpr (SUB == 1) {
      // two stages per iteration so that the roles of b0 and b1 are fixed
      int kt = 0;
      for (; kt + 2 <= nk; kt += 2) {
        step(acc, arena, kt, 0, b0, b1, a0, a1);
        step(acc, arena, kt + 1, 0, b1, b0, a0, a1);
      }
      if (kt < nk) step(acc, arena, kt, 0, b0, b1, a0, a1);
    } else {
      // SUB (even) K steps per stage: each but the last reads the next
      // step's fragments from the same buffer, the last waits for the next
      // stage
      static_assert(SUB % 2 == 0, "b0 / b1 alternate within a stage");
      for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
        for (int sub = 0; sub + 1 < SUB; ++sub) {
          if (sub % 2 == 0) first_half(acc, arena, kt, sub, b0, b1, a0, a1);
          else first_half(acc, arena, kt, sub, b1, b0, a0, a1);
        }
        step(acc, arena, kt, SUB - 1, b1, b0, a0, a1);
      }
    }
  }

  // K step `sub` of stage kt, not its last: its B blocks are in bc and its
  // first A block in a0; on return step sub + 1's are in bn and a0.
  __device__ __forceinline__ void first_half(f32x16_t (&acc)[NB][FM][FN], uint8_t* arena, int kt, int sub,
                                             BFrags& bc, BFrags& bn, AFrag& a0, AFrag& a1) const {
    const int buf = kt % NS;
#pragma unroll
    for (int i = 0; i + 1 < FM; ++i) {
      read_a(buf, i + 1, sub, arena, (i & 1) ? a0 : a1);
      __builtin_amdgcn_sched_barrier(0);
      mma_row<0, 1>(acc, i, (i & 1) ? a1 : a0, bc);
    }
    read_b(buf, sub + 1, arena, bn);
    read_a(buf, 0, sub + 1, arena, a0);
    __builtin_amdgcn_sched_barrier(0);
    mma_row<0, 1>(acc, FM - 1, a1, bc);
  }

  // Last K step `sub` of stage kt: its B blocks are in bc and its first A
  // block in a0; on return (unless it was the last stage) the next stage's
  // first step's are in bn and a0.
  __device__ __forceinline__ void step(f32x16_t (&acc)[NB][FM][FN], uint8_t* arena, int kt, int sub, BFrags& bc,
                                       BFrags& bn, AFrag& a0, AFrag& a1) const {
    const int buf = kt % NS;
#pragma unroll
    for (int i = 0; i + 1 < FM; ++i) {
      read_a(buf, i + 1, sub, arena, (i & 1) ? a0 : a1);
      __builtin_amdgcn_sched_barrier(0);
      mma_row<0, 1>(acc, i, (i & 1) ? a1 : a0, bc);
    }
    // the last row block is in a1 (FM even)
    if (kt + 1 < nk) {
      wait_stages<D, NS - 2>(nk - 2 - kt < NS - 2 ? nk - 2 - kt : NS - 2);
      read_b((kt + 1) % NS, 0, arena, bn);
      read_a((kt + 1) % NS, 0, 0, arena, a0);
      mma_issue<0, 4>(acc, a1, bc, kt + NS < nk, kt + NS, arena);
    } else {
      mma_row<0, 1>(acc, FM - 1, a1, bc);
    }
  }

  // DH: the saved A and B of a lane's 8 elements in each epilogue round
  // (round t: row block i = t / (2 FN), column block j = t / 2 % FN, half
  // t % 2), kept kPre rounds ahead in a ring of registers.  The first kPre
  // rounds are loaded before the next tile's stage copies are issued, so that
  // waiting for them does not wait for those copies too.
  static constexpr int kRounds = FM * FN * 2, kPre = 4;
  struct SavedPre {
    u32x4_t a[kPre], b[kPre];
  };
  __device__ __forceinline__ void dh_load(int t, SavedPre& p) const {
    const GroupedGemmArgs& a = *args;
    const int i = t / (2 * FN), j = (t / 2) % FN, half = t % 2;
    const int row = c.row0 + wm * TM + i * 32 + half * 16 + (lane >> 2);
    const int col = c.n0 + wn * TN + j * 32 + (lane & 3) * 8;
    const bool ok = row < c.row_end && col < N;
    const int64_t o = ok ? (int64_t)row * N + col : 0;
    p.a[t % kPre] = ok ? *reinterpret_cast<const u32x4_t*>((const bf16_t*)a.save_a + o) : u32x4_t{0u, 0u, 0u, 0u};
    p.b[t % kPre] = ok ? *reinterpret_cast<const u32x4_t*>((const bf16_t*)a.save_b + o) : u32x4_t{0u, 0u, 0u, 0u};
  }
  __device__ __forceinline__ void epilogue_prefetch(SavedPre& p) const {
    if constexpr (KIND == KIND_DH) {
#pragma unroll
      for (int t = 0; t < kPre; ++t) dh_load(t, p);
    }
  }

  // Epilogue through this wave's 4 KB of the staging area, 16 rows per round.
  __device__ __forceinline__ void epilogue(const f32x16_t (&acc)[NB][FM][FN], uint8_t* staging,
                                           SavedPre& pre) const {
    // The lane index passes through an empty asm so that the compiler cannot
    // compute the epilogue's per-lane addresses before the K loop (they would
    // stay live across it and push the loop into register spills).
    int lane = this->lane;
    asm volatile("" : "+v"(lane));
    float* ep = reinterpret_cast<float*>(staging + wid * 4096);
    const GroupedGemmArgs& a = *args;
    const int wrow0 = wm * TM, wcol0 = wn * TN;
    if constexpr (mx_wgrad<KIND>()) {
      // fp32 weight gradients straight from the accumulators: each half-wave
      // writes 32 consecutive floats of one row.  DW13: output rows below F
      // are dW1's, the rest dW3's (F is a multiple of 32, so a 32-row block
      // lies in one of them).
      (void)staging;
      (void)pre;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int m = c.m0 + wrow0 + i * 32;
        float* outp;
        int mr = m;
        if constexpr (KIND == KIND_DW13) {
          const bool w3 = m >= a.F;
          outp = (float*)(w3 ? a.out1 : a.out0);
          mr = w3 ? m - a.F : m;
        } else {
          outp = (float*)a.out0;
        }
        const int Mo = KIND == KIND_DW13 ? a.F : a.d;
        float* lp = outp + ((int64_t)c.e_loc * Mo + mr + (lane >> 5) * 4) * N + c.n0 + wcol0 + (lane & 31);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float* q = lp + (int64_t)((r >> 2) * 8 + (r & 3)) * N + j * 32;
            if constexpr (MOK_MXW_NT_STORE) __builtin_nontemporal_store(acc[0][i][j][r], q);
            else *q = acc[0][i][j][r];
          }
      }
    } else if constexpr (KIND == KIND_UP) {
      // gate and up of 16 rows x 32 columns per round; 4 consecutive lanes
      // hold the 32 columns (one MX block) of a row
      uint8_t* hq = (uint8_t*)a.out0;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
              const int rr = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);  // 0..15
              ep[rr * 32 + (lane & 31)] = acc[0][i][j][8 * half + r];
              ep[512 + rr * 32 + (lane & 31)] = acc[1][i][j][8 * half + r];
            }
            __builtin_amdgcn_wave_barrier();
            const int rr = lane >> 2, c8 = (lane & 3) * 8;
            const int row = c.row0 + wrow0 + i * 32 + half * 16 + rr, col = c.n0 + wcol0 + j * 32 + c8;
            const f32x4_t* pv = reinterpret_cast<const f32x4_t*>(&ep[rr * 32 + c8]);
            const f32x4_t* pu = reinterpret_cast<const f32x4_t*>(&ep[512 + rr * 32 + c8]);
            const f32x4_t v0 = pv[0], v1 = pv[1], u0 = pu[0], u1 = pu[1];
            const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            const float u[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
            float hv[8];
            float amax = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              hv[t] = v[t] * sigmoidf_(v[t]) * u[t];
              amax = fmaxf(amax, fabsf(hv[t]));
            }
            if (a.save && row < c.row_end && col < N) {
              // A, B and H before its quantisation, for the backward pass
              const int64_t o = (int64_t)row * N + col;
              *reinterpret_cast<u32x4_t*>((bf16_t*)a.save_a + o) = pack_bf16x8(v);
              *reinterpret_cast<u32x4_t*>((bf16_t*)a.save_b + o) = pack_bf16x8(u);
              *reinterpret_cast<u32x4_t*>((bf16_t*)a.out1 + o) = pack_bf16x8(hv);
            }
            amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
            amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
            const int se = FMT == kFmtE2M1 ? mx4_scale_exp(amax) : mx_scale_exp(amax);
            if (row < c.row_end && col < N) {
              if constexpr (FMT == kFmtE2M1) {
                *reinterpret_cast<uint32_t*>(hq + ((int64_t)row * N + col) / 2) = e2m1x8(hv, se);
              } else {
                const u32x2_t codes = pack_e4m3x8(hv, se);
                *reinterpret_cast<u32x2_t*>(hq + (int64_t)row * N + col) = codes;
              }
              if (c8 == 0) {
                const int b = col / 32;  // pair-plane layout of H's scales, P_max rows per plane
                a.out_scale[(int64_t)(b >> 1) * a.P_max * 2 + (int64_t)row * 2 + (b & 1)] = (uint8_t)(se + 127);
              }
            }
            __builtin_amdgcn_wave_barrier();
          }
    } else if constexpr (KIND == KIND_DH) {
      // dH of 16 rows x 32 columns per round; 4 consecutive lanes hold the 32
      // columns (one MX block) of a row.  With the saved A and B of those
      // elements: dA = dH * b * s (1 + a (1 - s)), dB = dH * a * s, s =
      // sigmoid(a); both written as bf16 into [dA | dB] (out0) and quantised
      // along F into out1 / out_scale (row r, block b: pair plane b / 2).
      bf16_t* dab = (bf16_t*)a.out0;
      uint8_t* dabq = (uint8_t*)a.out1;
      const int F2 = 2 * N;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
              const int rr = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);  // 0..15
              ep[rr * 32 + (lane & 31)] = acc[0][i][j][8 * half + r];
            }
            __builtin_amdgcn_wave_barrier();
            const int rr = lane >> 2, c8 = (lane & 3) * 8;
            const int row = c.row0 + wrow0 + i * 32 + half * 16 + rr, col = c.n0 + wcol0 + j * 32 + c8;
            const bool ok = row < c.row_end && col < N;
            const f32x4_t* pv = reinterpret_cast<const f32x4_t*>(&ep[rr * 32 + c8]);
            const f32x4_t v0 = pv[0], v1 = pv[1];
            const float dh[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            const int t = (i * FN + j) * 2 + half;
            const u32x4_t av = pre.a[t % kPre], bv = pre.b[t % kPre];
            if (t + kPre < kRounds) dh_load(t + kPre, pre);
            float da[8], db[8];
            float amax_a = 0.f, amax_b = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const uint32_t wa = av[t >> 1], wb = bv[t >> 1];
              const float x1 = __uint_as_float((t & 1) ? (wa & 0xFFFF0000u) : (wa << 16));
              const float x3 = __uint_as_float((t & 1) ? (wb & 0xFFFF0000u) : (wb << 16));
              const float sg = sigmoidf_(x1);
              da[t] = dh[t] * x3 * sg * (1.0f + x1 * (1.0f - sg));
              db[t] = dh[t] * x1 * sg;
              amax_a = fmaxf(amax_a, fabsf(da[t]));
              amax_b = fmaxf(amax_b, fabsf(db[t]));
            }
            amax_a = fmaxf(amax_a, __shfl_xor(amax_a, 1, 64));
            amax_a = fmaxf(amax_a, __shfl_xor(amax_a, 2, 64));
            amax_b = fmaxf(amax_b, __shfl_xor(amax_b, 1, 64));
            amax_b = fmaxf(amax_b, __shfl_xor(amax_b, 2, 64));
            const int sa = mx_scale_exp(amax_a), sb = mx_scale_exp(amax_b);
            if (ok) {
              bf16_t* drow = dab + (int64_t)row * F2;
              *reinterpret_cast<u32x4_t*>(drow + col) = pack_bf16x8(da);
              *reinterpret_cast<u32x4_t*>(drow + N + col) = pack_bf16x8(db);
              uint8_t* qrow = dabq + (int64_t)row * F2;
              *reinterpret_cast<u32x2_t*>(qrow + col) = pack_e4m3x8(da, sa);
              *reinterpret_cast<u32x2_t*>(qrow + N + col) = pack_e4m3x8(db, sb);
              if (c8 == 0) {
                const int ba = col / 32, bb = (N + col) / 32;
                a.out_scale[(int64_t)(ba >> 1) * a.P_max * 2 + (int64_t)row * 2 + (ba & 1)] = (uint8_t)(sa + 127);
                a.out_scale[(int64_t)(bb >> 1) * a.P_max * 2 + (int64_t)row * 2 + (bb & 1)] = (uint8_t)(sb + 127);
              }
            }
            __builtin_amdgcn_wave_barrier();
          }
    } else {
      // 16 rows x 64 columns per round, 8 lanes per row
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jp = 0; jp < FN / 2; ++jp)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
              for (int r = 0; r < 8; ++r) {
                const int rr = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                ep[rr * 64 + jj * 32 + (lane & 31)] = acc[0][i][2 * jp + jj][8 * half + r];
              }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const int seg = q * 64 + lane;
              const int rr = seg >> 3, c8 = (seg & 7) * 8;
              const int row = c.row0 + wrow0 + i * 32 + half * 16 + rr, col = c.n0 + wcol0 + jp * 64 + c8;
              if (row < c.row_end && col < N) {
                const f32x4_t* pv = reinterpret_cast<const f32x4_t*>(&ep[rr * 64 + c8]);
                const f32x4_t v0 = pv[0], v1 = pv[1];
                const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                u32x4_t y;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                  y[t] = (uint32_t)f2bf(v[2 * t]) | ((uint32_t)f2bf(v[2 * t + 1]) << 16);
                *reinterpret_cast<u32x4_t*>((bf16_t*)a.out0 + (int64_t)row * N + col) = y;
              }
            }
            __builtin_amdgcn_wave_barrier();
          }
    }
  }
};

// Persistent loop over the row tiles of the local experts (same order and
// XCD-aware mapping as the bf16 kernel); the next tile's first stages are
// issued before the current tile's epilogue.
template <int KIND, int NW, int FMT>
__global__ __launch_bounds__(NW * 64) void grouped_gemm_mxfp8_kernel(GroupedGemmArgs args) {
#if defined(__HIP_DEVICE_COMPILE__)
  using Job = MxJob<KIND, NW, FMT>;
  __shared__ __attribute__((aligned(1024))) uint8_t arena[Job::NS * Job::STAGE + Job::STAGING];
  uint8_t* const staging = arena + Job::NS * Job::STAGE;
  const int N = mx_n<KIND>(args.d, args.F);
  const int E_loc = args.E_loc;
  const int ntn = (N + Job::BN - 1) / Job::BN;
  const int32_t* tp = args.tile_prefix + 2 * (E_loc + 1);  // 256-row tiles
  const int total = sload(tp + E_loc) * ntn;
  const int G_ = gridDim.x;
  const int vb = (G_ % 8 == 0) ? (blockIdx.x % 8) * (G_ / 8) + blockIdx.x / 8 : blockIdx.x;
  auto coord = [&](int tile) -> TileCoord {
    const int q = tile / ntn;
    int lo = 0, hi = E_loc - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sload(tp + mid) <= q) lo = mid; else hi = mid - 1;
    }
    TileCoord c{};
    c.e_loc = lo;
    const int t0 = sload(tp + lo), t1 = sload(tp + lo + 1);
    int mt, nt;
    tile_mn<MOK_MX_GM>(tile - t0 * ntn, t1 - t0, ntn, mt, nt);
    c.n0 = nt * Job::BN;
    c.row0 = sload(args.offsets + args.eb + lo) + mt * Job::BM;
    c.row_end = sload(args.offsets + args.eb + lo + 1);
    return uniform(c);
  };
  int tile = vb;
  if (tile >= total) return;
  Job cur;
  cur.init(args, coord(tile));
  for (int s = 0; s < Job::NS && s < cur.nk; ++s) cur.issue(s, arena);
  f32x16_t acc[Job::NB][Job::FM][Job::FN];
  typename Job::SavedPre pre;
  while (true) {
    cur.mainloop(acc, arena);
    lds_barrier();  // every wave is done with the stage buffers
    cur.epilogue_prefetch(pre);
    const int nt = tile + G_;
    Job nxt = cur;
    if (nt < total) {
      nxt.init(args, coord(nt));
      for (int s = 0; s < Job::NS && s < nxt.nk; ++s) nxt.issue(s, arena);
    }
    cur.epilogue(acc, staging, pre);
    if (nt >= total) break;
    cur = nxt;
    tile = nt;
  }
#endif
}

// Weight-gradient kinds: every (local expert, 256-row, 128-column) tile of
// the output, experts taken heaviest first (the counting sort's rank order)
// so that the longest K loops start first, tiles of one expert in raster
// groups of two row tiles; a static round-robin over the persistent
// workgroups, XCD-contiguous as above.  Expert e's K range is its padded
// segment [128 tp128[e], 128 tp128[e + 1]) of the transposed operands.
template <int KIND, int NW>
__global__ __launch_bounds__(NW * 64) void grouped_wgrad_mxfp8_kernel(GroupedGemmArgs args) {
#if defined(__HIP_DEVICE_COMPILE__)
  using Job = MxJob<KIND, NW>;
  __shared__ __attribute__((aligned(1024))) uint8_t arena[Job::NS * Job::STAGE + Job::STAGING];
  uint8_t* const staging = arena + Job::NS * Job::STAGE;
  const int N = mx_n<KIND>(args.d, args.F), M = mx_m<KIND>(args.d, args.F);
  const int E_loc = args.E_loc;
  const int ntn = N / Job::BN, ntm = M / Job::BM;
  const int per_e = ntm * ntn;
  const int total = E_loc * per_e;
  const int32_t* tp = args.tile_prefix + 1 * (E_loc + 1);  // 128-row tiles: the padded segments
  const int G_ = gridDim.x;
  const int vb = (G_ % 8 == 0) ? (blockIdx.x % 8) * (G_ / 8) + blockIdx.x / 8 : blockIdx.x;
  auto coord = [&](int tile) -> TileCoord {
    TileCoord c{};
    const int rank = tile / per_e;
    c.e_loc = sload(args.expert_order + 4 * rank);
    c.row0 = 128 * sload(tp + c.e_loc);
    c.row_end = 128 * sload(tp + c.e_loc + 1);
    int mt, nt;
    tile_mn<2>(tile - rank * per_e, ntm, ntn, mt, nt);
    c.m0 = mt * Job::BM;
    c.n0 = nt * Job::BN;
    return uniform(c);
  };
  const int step = G_;
  auto valid = [&](int tile) { return tile < total; };
  int tile = vb;
  if (tile >= total) return;
  Job cur;
  cur.init(args, coord(tile));
  for (int s = 0; s < Job::NS && s < cur.nk; ++s) cur.issue(s, arena);
  f32x16_t acc[Job::NB][Job::FM][Job::FN];
  typename Job::SavedPre pre;
  while (true) {
    cur.mainloop(acc, arena);
    lds_barrier();  // every wave is done with the stage buffers
    const int nt = tile + step;
    const bool more = valid(nt);
    Job nxt = cur;
    if (more) {
      nxt.init(args, coord(nt));
      for (int s = 0; s < Job::NS && s < nxt.nk; ++s) nxt.issue(s, arena);
    }
    cur.epilogue(acc, staging, pre);
    if (!more) break;
    cur = nxt;
    tile = nt;
  }
#endif
}

template <int KIND, int NW>
static hipError_t run_mx_wgrad(const GroupedGemmArgs& g, hipStream_t s) {
  using Job = MxJob<KIND, NW>;
  const int N = mx_n<KIND>(g.d, g.F), M = mx_m<KIND>(g.d, g.F);
  if (N % Job::BN || M % Job::BM || g.k_pad % kMxBK) return hipErrorInvalidValue;
  const int64_t tiles = (int64_t)g.E_loc * (M / Job::BM) * (N / Job::BN);
  const int blocks = (int)(tiles < 256 ? tiles : 256);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_wgrad_mxfp8_kernel<KIND, NW>), dim3(blocks), dim3(NW * 64), 0, s, g);
  return hipGetLastError();
}

template <int KIND, int NW, int FMT = kFmtE4M3>
static hipError_t run_mx(const GroupedGemmArgs& g, hipStream_t s) {
  using Job = MxJob<KIND, NW, FMT>;
  const int N = mx_n<KIND>(g.d, g.F);
  if (mx_k<KIND>(g.d, g.F) % Job::KST) return hipErrorInvalidValue;
  const int ntn = (N + Job::BN - 1) / Job::BN;
  const int64_t worst = ((g.P_max + Job::BM - 1) / Job::BM + g.E_loc) * (int64_t)ntn;
  const int blocks = (int)(worst < 256 ? worst : 256);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_mxfp8_kernel<KIND, NW, FMT>), dim3(blocks), dim3(NW * 64), 0, s, g);
  return hipGetLastError();
}

hipError_t gemm_mxfp8(int kind, const GroupedGemmArgs& g, hipStream_t s) {
  switch (kind) {
    case KIND_UP:   return run_mx<KIND_UP, kMxWaves>(g, s);
    case KIND_DOWN: return run_mx<KIND_DOWN, kMxWaves>(g, s);
    case KIND_DH:   return run_mx<KIND_DH, kMxWaves>(g, s);
    case KIND_DX:   return run_mx<KIND_DX, kMxWaves>(g, s);
    case KIND_DW2:  return run_mx_wgrad<KIND_DW2, kMxWaves>(g, s);
    case KIND_DW13: return run_mx_wgrad<KIND_DW13, kMxWaves>(g, s);
  }
  return hipErrorNotSupported;
}

hipError_t gemm_mxfp4(int kind, const GroupedGemmArgs& g, hipStream_t s) {
  switch (kind) {
    case KIND_UP:   return run_mx<KIND_UP, kMxWaves, kFmtE2M1>(g, s);
    case KIND_DOWN: return run_mx<KIND_DOWN, kMxWaves, kFmtE2M1>(g, s);
  }
  return hipErrorNotSupported;
}

}  // namespace mok
