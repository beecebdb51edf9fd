// Host-side launchers of the MoE layer kernels and the buffer layouts they
// share.  Internal to libmok; the public interface is include/mok.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mok {

// Pairs handled by one wave in the counting sort.
constexpr int kSortChunk = 512;
// Row-tile heights for which per-expert tile prefixes are precomputed.
constexpr int kNumTileBM = 4;
constexpr int kTileBM[kNumTileBM] = {64, 128, 256, 32};
// The weight-streaming forward GEMMs take 32-row tiles (table 3).
constexpr int kStreamTileTable = 3;
constexpr int kStreamTileRows = 32;
constexpr int kNumCUs = 256;  // MI355X compute units

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct WorkspaceLayout {
  size_t status;        // uint32 device status word
  size_t chunk_counts;  // int32 [nchunks, E]
  size_t chunk_base;    // int32 [nchunks, E]
  size_t tile_prefix;   // int32 [kNumTileBM, E_loc + 1]
  size_t xp;            // dispatched rows: act [rows, d] or e4m3 [rows, d]
  size_t xp_scale;      // MXFP8: e8m0 [rows, d/32]
  size_t hq;            // MXFP8: e4m3 [P_max, F]
  size_t hq_scale;      // MXFP8: e8m0 [P_max, F/32]
  size_t dy;            // backward: act [P_max, d]
  size_t dab;           // backward: act [P_max, 2F]  (dA | dB)
  size_t dxp;           // backward: act [P_max, d]
  size_t queue;         // int32 tile counters of the weight-gradient GEMMs
  size_t wq;            // MXFP8 weight gradients: row-quantised transposed codes,
                        // [d | F | 2F | d] rows of k_pad bytes (dY, H, dA|dB, X)
  size_t wq_scale;      // their E8M0 scales, pair planes [k_pad / 64, C, 2] each
  int64_t k_pad;        // padded rows: 128 (P_max / 128 + E_loc), 0 without MXFP8 weight gradients
  size_t total;
  int nchunks;
  int64_t xp_rows;      // rows held by the dispatch buffer (P_max, or the ring)
};

// ----------------------------------------------------------------- launchers
// Router variant: bit 0 = sigmoid affinities (else softmax), bit 1 = gates
// renormalised over the chosen experts.
constexpr int kGateSigmoid = 1, kGateRenorm = 2;

// Status word (two int32 at the start of the workspace): cleared by
// launch_status_reset at the start of a call; kernels with device-side checks
// set it (mok_device.h report()).
hipError_t launch_status_reset(int32_t* status, hipStream_t s);

hipError_t launch_router_topk(const float* logits, int T, int E, int k, int gating, int32_t* idx_out,
                              float* gate_out, int32_t* idx_saved, float* gate_saved, float* lse,
                              int32_t* status, hipStream_t s);

// Small-T path: status reset, router and counting sort in one single-workgroup
// launch, for 1 <= T <= kSmallTokens and T * k <= kSmallPairs; the same
// outputs as launch_status_reset + launch_router_topk + launch_counting_sort.
// The 16 waves of the one workgroup route two tokens each at most: past that
// the router's arithmetic on one compute unit costs more than the launches
// saved.
constexpr int kSmallTokens = 32;
constexpr int kSmallPairs = 4096;
hipError_t launch_route_sort_small(const float* logits, int T, int E, int k, int gating, int eb, int ee,
                                   int32_t* idx_out, float* gate_out, int32_t* idx_saved, float* gate_saved,
                                   float* lse, int32_t* counts_out, int32_t* offsets_out, int32_t* offsets_saved,
                                   int32_t* tile_prefix, int32_t* expert_order, int32_t* row_of_pair,
                                   int32_t* pair_of_row, int32_t* status, hipStream_t s);

// MXFP8 quantisation of bf16 [rows, C] matrices along their rows, per local
// expert in blocks of 32 from the expert's first row, written transposed:
// codes [C, P_pad] at column 128 tp128[e] + (r - offsets[e]), scales in pair
// planes [P_pad / 64, C, 2].  Row r of a job is src row r (row stride ld
// elements), or with `gather` src row gather[r] / k_top, times gate[gather[r]]
// and rounded to bf16 when `gate` is set.  C a multiple of 64, P_pad of 128
// and at least 128 (P_max / 128 + E_loc).  All jobs in one launch.
constexpr int kQrMaxJobs = 4;
struct QrJob {
  const uint16_t* src;  // bf16
  int64_t ld;
  const int32_t* gather;
  const float* gate;
  int C;
  uint8_t* dst;
  uint8_t* dsc;
};
hipError_t launch_quantize_rows_t(const QrJob* jobs, int njobs, int k_top, const int32_t* offsets, int eb,
                                  int E_loc, const int32_t* tp128, int64_t P_max, int64_t P_pad, hipStream_t s);

hipError_t launch_counting_sort(const int32_t* idx, int T, int k, int E, int eb, int ee,
                                int nchunks, int32_t* chunk_counts, int32_t* chunk_base,
                                int32_t* counts_out, int32_t* offsets_out, int32_t* offsets_saved,
                                int32_t* tile_prefix, int32_t* expert_order, int32_t* row_of_pair,
                                int32_t* pair_of_row, hipStream_t s);

// X_perm[row(t,j)] = x[t] (act = bf16 when bf16 != 0, else fp32).  Row-map
// entries outside [-1, xp_rows) are reported on `status` and skipped.
hipError_t launch_dispatch_gather(const void* x, const int32_t* row_of_pair, int T, int k, int d,
                                  int bf16, void* xp, int64_t xp_rows, int32_t* status, hipStream_t s);
// Same, quantising each row to MXFP8 (E4M3 + E8M0 per 32 along d).
hipError_t launch_dispatch_gather_mxfp8(const void* x, const int32_t* row_of_pair, int T, int k,
                                        int d, uint8_t* xq, uint8_t* xs, int64_t xs_rows, int32_t* status,
                                        hipStream_t s);
hipError_t launch_quantize_mxfp8(const void* src, int64_t rows, int64_t K, uint8_t* q,
                                 uint8_t* sc, hipStream_t s);
// MXFP4: E2M1 codes two per byte (the lower element in the low nibble), xq
// rows of d / 2 bytes; scales in the same pair planes as MXFP8.
hipError_t launch_dispatch_gather_mxfp4(const void* x, const int32_t* row_of_pair, int T, int k,
                                        int d, uint8_t* xq, uint8_t* xs, int64_t xs_rows, int32_t* status,
                                        hipStream_t s);
hipError_t launch_quantize_mxfp4(const void* src, int64_t rows, int64_t K, uint8_t* q,
                                 uint8_t* sc, hipStream_t s);
// MXFP8 of the transpose of nmat [R, C] bf16 matrices along R (R, C multiples
// of 64): row c of matrix m at q + m q_mat + c q_ld + q_koff, scales in pair
// planes of `rows` rows, global row m C + c, K step (q_koff + r) / 64.
hipError_t launch_quantize_mxfp8_t(const void* src, int nmat, int R, int C, uint8_t* q, int64_t q_mat,
                                   int64_t q_ld, int q_koff, uint8_t* sc, int64_t rows, hipStream_t s);

// out[t] = sum_j w[t,j] * rows[row(t,j)] (w = gate, or 1 when gate == nullptr).
// all_local: the call owns every expert (else the kernel for mostly remote slots).
// Row-map entries outside [-1, nrows) are reported on `status` and skipped.
hipError_t launch_combine(const void* rows, const float* gate, const int32_t* row_of_pair, int T,
                          int k, int d, int bf16, int all_local, void* out, int64_t nrows, int32_t* status,
                          hipStream_t s);

// Reverse-combine and router backward: dgate, dlogits and dY rows.
hipError_t launch_backward_gate(const void* dout, const void* Y, const float* gate,
                                const int32_t* idx, const int32_t* row_of_pair,
                                const float* logits, const float* lse, int T, int k, int E, int d,
                                int gating, int bf16, float* dgate, float* dlogits, void* dy,
                                int32_t* queue_zero, int nqueue, uint8_t* dyq, uint8_t* dys,
                                int64_t dys_rows, int64_t nrows, int32_t* status, hipStream_t s);

// Grouped GEMMs of the expert FFN.  `offsets` is the global [E+1] array,
// experts [eb, eb + E_loc) are local.  tile_prefix is the [kNumTileBM, E_loc+1]
// table written by the counting sort.
struct GroupedGemmArgs {
  const void* A;          // activations (rows grouped by expert)
  const void* B0;         // per-expert weights
  const void* B1;         // second weights (W3) where used
  const int32_t* offsets;
  const int32_t* tile_prefix;
  const int32_t* expert_order;  // int4 per rank (heaviest first): {expert, row0, row_end, work prefix}
  int32_t* queue;               // 8 per-XCD tile counters of a weight-gradient kind (zeroed on device)
  int eb, E_loc;
  int d, F;
  int64_t P_max;
  void* out0;             // H / Y / dAB / dXp / dW
  void* out1;             // second output where used (dW3)
  void* save_a;           // A (pre-activation) rows
  void* save_b;           // B rows
  const uint8_t* a_scale; // MXFP8 activation scales
  const uint8_t* b_scale0;
  const uint8_t* b_scale1;
  uint8_t* out_scale;     // MXFP8 H scales
  int save;               // write A and B (forward)
  // Pull dispatch fused into the GEMM loads: when non-null, row r of the
  // expert-sorted operand (A of UP; B of DW13 in ring mode) is row
  // gather_rows[r] / k_top of the token matrix (x, with gather_src_rows rows).
  const int32_t* gather_rows;
  int k_top;
  int64_t gather_src_rows;
  // Ring mode: the A operand of UP holds row r at A row r - a_row_shift.
  int64_t a_row_shift;
  // MXFP8 weight gradients: row stride (bytes) of the transposed, row-quantised
  // operands; expert e's K range is [128 tp128[e], 128 tp128[e + 1]).
  int64_t k_pad;
};

// Expert-grouped GEMM of one kind (GemmKind in gemm_common.h) per precision:
// 0 UP (H = silu(X W1^T) * (X W3^T)), 1 DOWN (Y = H W2^T), 2 DH (dA, dB from
// dY W2), 3 DX (dA W1 + dB W3), 4 DW2 (dY^T H), 5 DW13 (dA^T X, dB^T X).
hipError_t gemm_bf16(int kind, const GroupedGemmArgs& g, hipStream_t s);

// Weight-streaming bf16 UP and DOWN for calls with few rows per expert: one
// workgroup per (32-row tile, 16-64 weight rows) unit, the weight rows read
// once per tile straight into registers, 16x16x32 MFMA.  Same arguments and
// outputs as gemm_bf16's UP (with pull dispatch: gather_rows set) and DOWN.
// stream_ksplit(K): the waves splitting K (4, 2 or 1), 0 when K is not a
// multiple of 128 (then only the tiled kernels apply).
int stream_ksplit(int K);
hipError_t gemm_stream_bf16(int kind, const GroupedGemmArgs& g, hipStream_t s);
// The MXFP8 forward's UP (E4M3 x rows from the dispatch, H quantised along F)
// and DOWN (bf16 Y) the same way, on the 32x32x64 scaled MFMA: 32-row tiles,
// 32-column units; forward only.  stream_mx_ok: d % 256 == 0, F % 128 == 0.
int stream_mx_ok(int d, int F);
hipError_t gemm_stream_mxfp8(int kind, const GroupedGemmArgs& g, hipStream_t s);
// The same with E2M1 operands (MXFP4 forward): d % 256 == 0, F % 128 == 0.
hipError_t gemm_stream_mxfp4(int kind, const GroupedGemmArgs& g, hipStream_t s);

// One step of the ring-buffer minibatch pipeline (bf16): in a single launch,
// mover tiles copy the rows of minibatch m+1 into their ring slot, compute
// tiles run UP on minibatch m (rows read from its ring slot) and DOWN on
// minibatch m-1.  Row ranges are half-open in the expert-sorted row space and
// are clipped on the device to the local row count.
struct MinibatchStepArgs {
  GroupedGemmArgs up;     // A = ring (a_row_shift maps row r to its slot row)
  GroupedGemmArgs down;   // A = H
  int up0, up1;           // rows of minibatch m   (up0 == up1: none)
  int dn0, dn1;           // rows of minibatch m-1 (dn0 == dn1: none)
  int cp0, cp1;           // rows of minibatch m+1 to copy (cp0 == cp1: none)
  const void* x;          // [T, d] bf16 token rows
  const int32_t* pair_of_row;
  int k;
  void* ring_dst;         // ring slot receiving row cp0
  int movers;             // workgroups that only copy (0: one queue for every task)
  int32_t* ctr;           // kRingCounters task counters, zero before the launch and left zero by it
};
constexpr int kRingCounters = 9;  // one per XCD run, and the count of finished workgroups
hipError_t launch_minibatch_step(const MinibatchStepArgs& a, hipStream_t s);
// Zeroes the ring kernel's task counters (before the first launch of a call).
hipError_t launch_ring_reset(int32_t* ctr, hipStream_t s);
hipError_t gemm_f32(int kind, const GroupedGemmArgs& g, hipStream_t s);
hipError_t gemm_mxfp8(int kind, const GroupedGemmArgs& g, hipStream_t s);
// MXFP4 forward (inference) UP and DOWN: the MXFP8 kernels with E2M1 operands
// (two codes per byte, activations as written by launch_dispatch_gather_mxfp4,
// H quantised to MXFP4 along F in UP's epilogue); K a multiple of 256.
hipError_t gemm_mxfp4(int kind, const GroupedGemmArgs& g, hipStream_t s);

}  // namespace mok
