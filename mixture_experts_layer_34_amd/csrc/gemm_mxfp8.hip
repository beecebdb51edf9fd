// Expert-grouped MXFP8 GEMMs (gfx950 v_mfma_scale_f32_32x32x64_f8f6f4), forward:
//   UP    H_e = silu(X_e W1_e^T) * (X_e W3_e^T), quantised to MXFP8 along F
//   DOWN  Y_e = H_e W2_e^T (bf16)
// Operands are E4M3 with one E8M0 scale per 32 consecutive K values (OCP MX
// v1.0).  MXFP8 activation quantisation sits in the dispatch, grouped-GEMM and
// SwiGLU data paths instead of a standalone kernel (kucoin.com, "Cursor's MoK
// réalise une amélioration des performances de 2,37x sur NVIDIA GB300 NVL72",
// section 02): X rows are quantised by the dispatch gather, H by this UP
// epilogue, and the scaled MFMA consumes both without dequantising.
//
// A K step is 128 fp8 values = 128 bytes per row, so the LDS tiles, the XOR
// swizzle, the direct-to-LDS loads and the tile scheduling are those of the
// BF16 kernel.  Scaled-MFMA operand layout on gfx950 (checked on the device):
// for each 64-wide K sub-step, lane l holds row l % 32; with h = l / 32 its
// bytes 0-15 are K [16h, 16h + 16) and bytes 16-31 are K [32 + 16h, +16), and
// the scale it supplies covers the 32-block h of the sub-step.
#include "mok_device.h"
#include "mok_internal.h"
#include "gemm_common.h"

namespace mok {

namespace {

[[maybe_unused]] constexpr int kBKq = 128;          // K per stage (fp8 elements = bytes)
[[maybe_unused]] constexpr int kRowB = 128;         // LDS row bytes

[[maybe_unused]] __device__ __forceinline__ int swzq(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

[[maybe_unused]] __device__ __forceinline__ void tile_mn_q(int local, int mt, int ntn, int& m, int& n) {
  constexpr int GM = 4;
  const int g = local / (GM * ntn);
  const int gm0 = g * GM;
  const int gsz = mt - gm0 < GM ? mt - gm0 : GM;
  const int rem = local - g * GM * ntn;
  n = rem / gsz;
  m = gm0 + rem % gsz;
}

}  // namespace

template <int KIND, int BM, int BN>
__global__ __launch_bounds__(256) void grouped_gemm_mxfp8_kernel(GroupedGemmArgs args) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NB = KIND == KIND_UP ? 2 : 1;
  constexpr int BROWS = NB * BN;
  constexpr int TM = BM / 2, TN = BN / 2, FM = TM / 32, FN = TN / 32;
  constexpr int DMA_A = BM / 8 / 4, DMA_B = BROWS / 8 / 4;
  constexpr int kArena = 2 * (BM + BROWS) * kRowB;
  static_assert(kArena >= 4 * 32768, "epilogue staging needs 32 KB per wave");
  __shared__ __attribute__((aligned(1024))) uint8_t arena[kArena];
  __shared__ int32_t s_tp[1025];
  uint8_t (*sA)[BM * kRowB] = reinterpret_cast<uint8_t (*)[BM * kRowB]>(arena);
  uint8_t (*sB)[BROWS * kRowB] = reinterpret_cast<uint8_t (*)[BROWS * kRowB]>(arena + 2 * BM * kRowB);

  // K (contraction) and N (output columns) of this kind
  const int K = KIND == KIND_UP ? args.d : args.F;
  const int N = KIND == KIND_UP ? args.F : args.d;
  const int KS = K / 32;                      // scale bytes per row
  const int64_t b_estride = (int64_t)args.F * args.d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps DMA operands scalar
  const int wm = wid / 2, wn = wid % 2;
  const uint8_t* __restrict__ A = (const uint8_t*)args.A;
  const uint8_t* __restrict__ B0 = (const uint8_t*)args.B0;
  const uint8_t* __restrict__ B1 = (const uint8_t*)args.B1;
  const int E_loc = args.E_loc;
  const int ntn = (N + BN - 1) / BN;

  const int32_t* tp = args.tile_prefix + 2 * (E_loc + 1);  // 256-row tiles
  for (int i = tid; i <= E_loc; i += 256) s_tp[i] = tp[i];
  __syncthreads();
  const int total = s_tp[E_loc] * ntn;
  const int G_ = gridDim.x;
  const int vb = (G_ % 8 == 0) ? (blockIdx.x % 8) * (G_ / 8) + blockIdx.x / 8 : blockIdx.x;

  for (int tile = vb; tile < total; tile += G_) {
    int lo = 0, hi = E_loc - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (s_tp[mid] * ntn <= tile) lo = mid; else hi = mid - 1;
    }
    int e_loc = lo, mt, nt;
    tile_mn_q(tile - s_tp[e_loc] * ntn, s_tp[e_loc + 1] - s_tp[e_loc], ntn, mt, nt);
    int n0 = nt * BN;
    int row0 = args.offsets[args.eb + e_loc] + mt * BM;
    int row_end = args.offsets[args.eb + e_loc + 1];
    e_loc = __builtin_amdgcn_readfirstlane(e_loc);
    n0 = __builtin_amdgcn_readfirstlane(n0);
    row0 = __builtin_amdgcn_readfirstlane(row0);
    row_end = __builtin_amdgcn_readfirstlane(row_end);
    const int nk = K / kBKq;

    // direct-to-LDS sources (rows past the tile's data read as zero)
    const int rows = row_end - row0 < BM ? row_end - row0 : BM;
    const i32x4_t rsA = make_rsrc(A + (int64_t)row0 * K, (uint32_t)(rows * K));
    const int nb_rows = N - n0 < BN ? N - n0 : BN;
    const uint8_t* b0 = B0 + (int64_t)e_loc * b_estride + (int64_t)n0 * K;
    const i32x4_t rsB0 = make_rsrc(b0, (uint32_t)(nb_rows * K));
    const uint8_t* b1 = (NB == 2 ? B1 : B0) + (int64_t)e_loc * b_estride + (int64_t)n0 * K;
    const i32x4_t rsB1 = make_rsrc(b1, (uint32_t)(nb_rows * K));
    uint32_t offA[DMA_A], offB[DMA_B];
#pragma unroll
    for (int q = 0; q < DMA_A; ++q) {
      const int r = (wid * DMA_A + q) * 8 + (lane >> 3);
      offA[q] = (uint32_t)(r * K + swzq(r, lane & 7) * 16);
    }
#pragma unroll
    for (int q = 0; q < DMA_B; ++q) {
      const int r = (wid * DMA_B + q) * 8 + (lane >> 3);
      const int rl = (NB == 2 && r >= BN) ? r - BN : r;
      offB[q] = (uint32_t)(rl * K + swzq(r, lane & 7) * 16);
    }
    // scale rows of this lane's fragments (clamped into the data rows)
    const uint8_t* sa_rows[FM];
    const uint8_t* sb_rows[NB][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      int r = row0 + wm * TM + i * 32 + (lane & 31);
      r = r < row_end ? r : row_end - 1;
      sa_rows[i] = args.a_scale + (int64_t)r * KS;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        int n = n0 + wn * TN + j * 32 + (lane & 31);
        n = n < N ? n : N - 1;
        sb_rows[b][j] = (b ? args.b_scale1 : args.b_scale0) + ((int64_t)e_loc * N + n) * KS;
      }
    const int hsh = 8 * (lane >> 5);  // this lane's scale byte within each pair of 32-blocks
    uint32_t scA[FM], scB[NB][FN];
    auto load_scales = [&](int k0) {
#pragma unroll
      for (int i = 0; i < FM; ++i) scA[i] = *reinterpret_cast<const uint32_t*>(sa_rows[i] + k0 / 32) >> hsh;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < FN; ++j) scB[b][j] = *reinterpret_cast<const uint32_t*>(sb_rows[b][j] + k0 / 32) >> hsh;
    };
    auto issue = [&](int k0, int buf) {
#pragma unroll
      for (int q = 0; q < DMA_A; ++q)
        dma_b128(rsA, lds_addr(&sA[buf][(wid * DMA_A + q) * 1024]), offA[q], k0);
#pragma unroll
      for (int q = 0; q < DMA_B; ++q) {
        dma_b128((NB == 2 && (wid * DMA_B + q) * 8 >= BN) ? rsB1 : rsB0,
                 lds_addr(&sB[buf][(wid * DMA_B + q) * 1024]), offB[q], k0);
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

    issue(0, 0);
    load_scales(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      uint32_t cA[FM], cB[NB][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) cA[i] = scA[i];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < FN; ++j) cB[b][j] = scB[b][j];
      if (kt + 1 < nk) {
        issue((kt + 1) * kBKq, buf ^ 1);
        load_scales((kt + 1) * kBKq);
      }
      const uint8_t* a_s = sA[buf];
      const uint8_t* b_s = sB[buf];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int c0 = ks * 4 + (lane >> 5), c1 = c0 + 2;
        i32x8_t af[FM], bfr[NB][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = wm * TM + i * 32 + (lane & 31);
          const u32x4_t lo4 = *reinterpret_cast<const u32x4_t*>(&a_s[r * kRowB + swzq(r, c0) * 16]);
          const u32x4_t hi4 = *reinterpret_cast<const u32x4_t*>(&a_s[r * kRowB + swzq(r, c1) * 16]);
          af[i] = i32x8_t{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                          (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int r = b * BN + wn * TN + j * 32 + (lane & 31);
            const u32x4_t lo4 = *reinterpret_cast<const u32x4_t*>(&b_s[r * kRowB + swzq(r, c0) * 16]);
            const u32x4_t hi4 = *reinterpret_cast<const u32x4_t*>(&b_s[r * kRowB + swzq(r, c1) * 16]);
            bfr[b][j] = i32x8_t{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3],
                                (int)hi4[0], (int)hi4[1], (int)hi4[2], (int)hi4[3]};
          }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              if (ks == 0)
                acc[b][i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bfr[b][j], acc[b][i][j], 0, 0,
                                                                                0, (int)cA[i], 0, (int)cB[b][j]);
              else
                acc[b][i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bfr[b][j], acc[b][i][j], 0, 0,
                                                                                2, (int)cA[i], 2, (int)cB[b][j]);
            }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue (LDS staged)
    float* ep = reinterpret_cast<float*>(arena + wid * 32768);
    const int wrow0 = wm * TM, wcol0 = wn * TN;
    if constexpr (KIND == KIND_UP) {
      uint8_t* hq = (uint8_t*)args.out0;
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
        // 4 consecutive lanes hold the 32 columns of one row's MX block
        for (int q = 0; q < TM * 32 / 8 / 64; ++q) {
          const int seg = q * 64 + lane;
          const int rr = seg >> 2, c8 = (seg & 3) * 8;
          const int row = row0 + wrow0 + rr, col = n0 + wcol0 + j * 32 + c8;
          const f32x4_t* pv = reinterpret_cast<const f32x4_t*>(&ep[rr * 32 + c8]);
          const f32x4_t* pu = reinterpret_cast<const f32x4_t*>(&ep[4096 + rr * 32 + c8]);
          const f32x4_t v0 = pv[0], v1 = pv[1], u0 = pu[0], u1 = pu[1];
          const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
          const float u[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
          float h[8];
          float amax = 0.f;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            h[t] = v[t] * sigmoidf_(v[t]) * u[t];
            amax = fmaxf(amax, fabsf(h[t]));
          }
          amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
          amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
          const int se = mx_scale_exp(amax);
          uint32_t c[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) c[t] = e4m3_rne(ldexpf(h[t], -se));
          if (row < row_end && col < N) {
            u32x2_t codes;
            codes[0] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
            codes[1] = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
            *reinterpret_cast<u32x2_t*>(hq + (int64_t)row * N + col) = codes;
            if (c8 == 0) args.out_scale[(int64_t)row * (N / 32) + col / 32] = (uint8_t)(se + 127);
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
          const int row = row0 + wrow0 + rr, col = n0 + wcol0 + jp * 64 + c8;
          if (row < row_end && col < N) {
            const f32x4_t* pv = reinterpret_cast<const f32x4_t*>(&ep[rr * 64 + c8]);
            const f32x4_t v0 = pv[0], v1 = pv[1];
            const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            u32x4_t y;
#pragma unroll
            for (int t = 0; t < 4; ++t) y[t] = (uint32_t)f2bf(v[2 * t]) | ((uint32_t)f2bf(v[2 * t + 1]) << 16);
            *reinterpret_cast<u32x4_t*>((bf16_t*)args.out0 + (int64_t)row * N + col) = y;
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
    __syncthreads();
  }
#endif
}

template <int KIND, int BM, int BN>
static hipError_t run_mx(const GroupedGemmArgs& g, hipStream_t s) {
  const int N = KIND == KIND_UP ? g.F : g.d;
  const int ntn = (N + BN - 1) / BN;
  const int64_t worst = ((g.P_max + BM - 1) / BM + g.E_loc) * (int64_t)ntn;
  const int blocks = (int)(worst < 256 ? worst : 256);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_mxfp8_kernel<KIND, BM, BN>), dim3(blocks), dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t gemm_mxfp8(int kind, const GroupedGemmArgs& g, hipStream_t s) {
  switch (kind) {
    case KIND_UP:   return run_mx<KIND_UP, 256, 128>(g, s);
    case KIND_DOWN: return run_mx<KIND_DOWN, 256, 256>(g, s);
  }
  return hipErrorNotSupported;
}

}  // namespace mok
