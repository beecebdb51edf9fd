/*
 * mok_diag.h — diagnostics of the matrix cores the MoE layer runs on
 * (libmok_diag.so, separate from the layer's libmok.so).  Test support only.
 */
#ifndef MOK_DIAG_H_
#define MOK_DIAG_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * One block of the gfx950 scaled matrix instruction the MXFP8 GEMMs use
 * (32 x 32 outputs, K = 64, E4M3 operands, one E8M0 scale per 32 K values of
 * each row; the MXFP8 format of kucoin.com, "Cursor's MoK réalise une
 * amélioration des performances de 2,37x sur NVIDIA GB300 NVL72", section 02):
 *   C_out[i][j] = C_in[i][j] + sum_{k < 64} A[i][k] 2^(sa[i][k/32] - 127)
 *                                          * B[j][k] 2^(sb[j][k/32] - 127)
 * as the hardware computes it, so that a caller can compare it with the
 * exact sum.
 *   a, b        device, uint8 [32][64] E4M3 codes (rows i of A, rows j of B)
 *   sa, sb      device, uint8 [32][2] E8M0 scale bytes
 *   c_in, c_out device, float [32][32], row-major
 * One wave on `stream` (a hipStream_t as void*); returns 0, 1 for a null
 * pointer, 4 for a failed launch.
 */
int32_t mok_diag_mfma_scale_block(const uint8_t* a, const uint8_t* b, const uint8_t* sa, const uint8_t* sb,
                                  const float* c_in, float* c_out, void* stream);

/*
 * The same instruction on raw operand registers, for establishing its
 * register-to-K mapping per operand format: lane l (0..63) supplies A dwords
 * a[8 l .. 8 l + 7], B dwords b[8 l .. 8 l + 7], scale bytes sa[l], sb[l] and
 * accumulators c_in[16 l .. 16 l + 15]; c_out[16 l + i] is its result
 * register i.  fmt_a / fmt_b: 0 = E4M3, 4 = E2M1 (FP4 codes; the instruction
 * then reads the first four dwords of each lane); supported pairs (0, 0),
 * (4, 4) and (4, 0).  All pointers device memory.  One wave on `stream`;
 * returns 0, 1 for a null pointer or an unsupported pair, 4 for a failed
 * launch.
 */
int32_t mok_diag_mfma_scale_raw(const uint32_t* a, const uint32_t* b, const uint8_t* sa, const uint8_t* sb,
                                const float* c_in, float* c_out, int32_t fmt_a, int32_t fmt_b, void* stream);

/*
 * The E4M3 encoding the layer's MXFP8 quantisers use (the gfx950 conversion
 * instruction on the value clamped to +-448, one value and four packed
 * little-endian) against a software encoder written from the OCP E4M3
 * definition (round to nearest even, saturation to +-448, sign of zero kept),
 * over every float32 bit pattern u < n and its negation (n <= 0x44000000,
 * the magnitudes below 2^9 that scaled MX elements take).
 *   count, first  device, uint32 [blocks * 256]: per thread, the number of
 *                 mismatching values and the first one's bit pattern
 *                 (0xFFFFFFFF when none)
 * Returns 0, 1 for a null pointer or an out-of-range n or blocks, 4 for a
 * failed launch.
 */
int32_t mok_diag_e4m3_check(uint32_t n, uint32_t* count, uint32_t* first, int32_t blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOK_DIAG_H_ */
