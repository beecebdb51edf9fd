// MXFP8 quantisation along the token axis, for the MXFP8 weight-gradient
// GEMMs (dW2 = Qr(dY)^T Qr(H), dW1 = Qr(dA)^T Qr(X), dW3 = Qr(dB)^T Qr(X)):
// their contraction runs over an expert's rows, so every operand is cut, per
// column, into blocks of 32 consecutive rows from the expert's first row
// (placement order), the last block of a segment taking its scale from the
// rows it has.  The codes are written transposed, K-contiguous per column,
// so that the scaled-MFMA kernels read them like any K-contiguous operand:
//   codes[c][pos]  pos = 128 tp128[e] + (row - offsets[e]), E4M3
//   scales         pair planes: byte (pos / 64, c, pos / 32 % 2) at
//                  (pos / 64) * 2 C + 2 c + pos / 32 % 2, E8M0
// where tp128 is the counting sort's 128-row tile prefix, so each expert's
// segment starts on a 128-row boundary; rows past the expert up to that
// boundary hold zero codes (and their all-zero blocks scale byte 0).  Block
// scale: 2^(floor(log2 amax) - 8), elements E4M3(v / scale), round to nearest
// even, saturating (OCP MX v1.0; the same encoder as the other MXFP8 paths).
#include "mok_device.h"
#include "mok_internal.h"
#include "gemm_pipe.h"

namespace mok {
namespace {

constexpr int kQrRows = 128;  // rows per unit (one padded K stage of the GEMMs)
constexpr int kQrCols = 64;   // columns per unit
static_assert(kQrMaxJobs >= 4, "dY, H, [dA | dB] and x in one launch");

// One workgroup of 256 threads per (matrix, 128-row block of a local
// expert's padded segment, 64 columns) unit, persistent over the units of all
// the matrices of one launch.  The block's rows come in coalesced (16 bytes
// per thread, 8 threads per 128-byte row piece) into LDS; thread (c = tid /
// 4, b = tid % 4) then takes column c of the block's 32-row sub-block b:
// amax, scale, 32 codes (two 16-byte stores), so that the four threads of a
// column, adjacent lanes, write its 128 bytes of the block together.  In LDS
// the 16-byte column chunks of row r are XOR-ed with its sub-block (r / 32)
// so that those four threads, reading the same column of rows 32 apart, hit
// different banks.  A gated matrix (dY) is formed while loading: row r is
// bf16(gate[p] * src[p / k]), p = gather[r], the same product and rounding
// as the reverse-combine's dY rows.
struct QrJobs {
  QrJob job[kQrMaxJobs];
  int njobs, k_top, eb, E_loc;
  const int32_t* offsets;
  const int32_t* tp128;
  int64_t P_pad;
};

__global__ __launch_bounds__(256) void quantize_rows_t_kernel(QrJobs a) {
  __shared__ bf16_t tile[kQrRows][kQrCols];
  const int tid = threadIdx.x;
  const int nblk = sload(a.tp128 + a.E_loc);
  int total = 0;
  for (int j = 0; j < a.njobs; ++j) total += nblk * (a.job[j].C / kQrCols);
  for (int u = blockIdx.x; u < total; u += gridDim.x) {
    int j = 0, uj = u;
    while (uj >= nblk * (a.job[j].C / kQrCols)) {
      uj -= nblk * (a.job[j].C / kQrCols);
      ++j;
    }
    const QrJob& jb = a.job[j];
    const int ncb = jb.C / kQrCols;
    const int t = uj / ncb, cb = uj % ncb;
    int lo = 0, hi = a.E_loc - 1;  // the local expert whose 128-row blocks hold t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sload(a.tp128 + mid) <= t) lo = mid; else hi = mid - 1;
    }
    const int blk = t - sload(a.tp128 + lo);
    const int r0 = sload(a.offsets + a.eb + lo) + blk * kQrRows;
    const int rend = sload(a.offsets + a.eb + lo + 1);
    const int c0 = cb * kQrCols;
    __syncthreads();  // the previous unit's tile is read
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int q = tid + 256 * q4;
      const int rr = q >> 3, ch = q & 7;
      const int row = r0 + rr;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row < rend) {
        int64_t srow = row;
        float g = 1.0f;
        if (jb.gather) {
          const int p = jb.gather[row];
          srow = p / a.k_top;
          if (jb.gate) g = jb.gate[p];
        }
        v = *reinterpret_cast<const u32x4_t*>(jb.src + srow * jb.ld + c0 + ch * 8);
        if (jb.gate) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float lo_ = g * __uint_as_float(v[i] << 16), hi_ = g * __uint_as_float(v[i] & 0xFFFF0000u);
            v[i] = (uint32_t)f2bf(lo_) | ((uint32_t)f2bf(hi_) << 16);
          }
        }
      }
      *reinterpret_cast<u32x4_t*>(&tile[rr][(ch ^ (rr >> 5)) * 8]) = v;
    }
    __syncthreads();
    const int c = tid >> 2, b = tid & 3;
    const int cs = c ^ (8 * b);  // the column's place in rows of sub-block b
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      v[i] = bf2f(tile[32 * b + i][cs]);
      amax = fmaxf(amax, fabsf(v[i]));
    }
    const int se = mx_scale_exp(amax);
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      w[q] = e4m3x4(ldexpf(v[4 * q], -se), ldexpf(v[4 * q + 1], -se), ldexpf(v[4 * q + 2], -se),
                    ldexpf(v[4 * q + 3], -se));
    const int64_t pos = (int64_t)t * kQrRows + 32 * b;
    uint8_t* out = jb.dst + (int64_t)(c0 + c) * a.P_pad + pos;
    *reinterpret_cast<u32x4_t*>(out) = u32x4_t{w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4_t*>(out + 16) = u32x4_t{w[4], w[5], w[6], w[7]};
    jb.dsc[(pos / 64) * 2 * jb.C + 2 * (c0 + c) + ((pos / 32) & 1)] = (uint8_t)(se + 127);
  }
}

}  // namespace

hipError_t launch_quantize_rows_t(const QrJob* jobs, int njobs, int k_top, const int32_t* offsets, int eb,
                                  int E_loc, const int32_t* tp128, int64_t P_max, int64_t P_pad, hipStream_t s) {
  if (njobs < 1 || njobs > kQrMaxJobs || P_pad % kQrRows) return hipErrorInvalidValue;
  QrJobs a{};
  int64_t cols = 0;
  for (int j = 0; j < njobs; ++j) {
    if (jobs[j].C % kQrCols || (jobs[j].gate && !jobs[j].gather)) return hipErrorInvalidValue;
    a.job[j] = jobs[j];
    cols += jobs[j].C / kQrCols;
  }
  a.njobs = njobs;
  a.k_top = k_top;
  a.eb = eb;
  a.E_loc = E_loc;
  a.offsets = offsets;
  a.tp128 = tp128;
  a.P_pad = P_pad;
  // units: at most (P_max / 128 + E_loc) blocks of 128 rows per 64 columns
  const int64_t worst = (P_max / kQrRows + E_loc) * cols;
  const int64_t cap = (int64_t)kNumCUs * 8;
  const int blocks = (int)(worst < cap ? worst : cap);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_rows_t_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mok
