/*
 * mok.h — C ABI of the fused, deterministic mixture-of-experts layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (forward): router softmax + stable top-k, counting-sort dispatch
 * of token-expert pairs into an expert-contiguous buffer, expert-grouped
 * SwiGLU FFN GEMMs (BF16, MXFP8 or FP32), and a gate-weighted combine in a
 * fixed summation order.  Backward mirrors it and returns dX, dW1/dW3/dW2,
 * d(gate) and d(router logits).
 *
 * Pages this interface follows (cited by title and section):
 *   [kucoin] kucoin.com, "Cursor's MoK réalise une amélioration des
 *            performances de 2,37x sur NVIDIA GB300 NVL72", sections 01-03;
 *   [fluid]  fluidifia.com, "Cursor ouvre MoK, un mégakernel qui accélère
 *            l'entraînement MoE";
 *   [ixtr]   ixtr.ca, "Introduction à Mixture-of-Kittens", section
 *            "Écosystème Logiciel" (a light package exposing the kernel API
 *            as a drop-in MoE routine);
 *   [martel] laura-martel.com post on Mixture-of-Kittens, sections "Ce qu'il
 *            fait réellement" (one kernel, one launch, no host round trip
 *            inside the layer) and "Le déterminisme est la partie
 *            sous-estimée" (same inputs, same hardware, same result).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates or frees device memory and never synchronises
 *     the host: every call validates its arguments on the host, enqueues its
 *     kernels on `stream` (a hipStream_t passed as void*, NULL = the default
 *     stream) and returns.  Outputs are valid once the stream reaches them.
 *   - Row-major layouts.  T tokens, hidden size d, E experts, top-k k,
 *     expert FFN width F (cfg->ffn).  Local experts are
 *     [expert_begin, expert_end); E_loc = expert_end - expert_begin and the
 *     weights of expert e sit at index e - expert_begin.
 *   - Activation element type: bf16 for MOK_PREC_BF16, MOK_PREC_MXFP8 and
 *     MOK_PREC_MXFP4 (x, out, dout, dx), fp32 for MOK_PREC_F32.
 *   - Pair id p = t*k + j (slot j = 0 is the highest-ranked expert).
 *   - Errors: a non-MOK_OK status is returned and nothing is enqueued.
 *     No exception crosses the ABI.  Results are bit-identical from run to
 *     run for identical inputs on the same device [martel].
 *   - T = 0 is valid: counts and offsets become 0, dW outputs 0; pointers
 *     to arrays with zero elements may be NULL.
 */
#ifndef MOK_H_
#define MOK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOK_OK = 0,
  MOK_ERR_INVALID_ARG = 1,   /* null pointer, bad shape, misalignment          */
  MOK_ERR_UNSUPPORTED = 2,   /* valid request this build does not implement     */
  MOK_ERR_WORKSPACE = 3,     /* ring smaller than two minibatch slots           */
  MOK_ERR_HIP = 4,           /* a HIP runtime call failed (launch error)        */
  MOK_ERR_DEVICE = 5         /* reported by a device-side check                 */
} mok_status;

typedef enum {
  MOK_PREC_F32 = 0,          /* fp32 activations and weights, fp32 arithmetic   */
  MOK_PREC_BF16 = 1,         /* bf16 operands, fp32 accumulation (MFMA)         */
  MOK_PREC_MXFP8 = 2,        /* E4M3 operands + E8M0 scale per 32 along K       */
  MOK_PREC_MXFP4 = 3         /* E2M1 operands + E8M0 scale per 32 along K;
                                forward only (see mok_moe_forward)              */
} mok_precision;

/* Forward writes the intermediates backward needs (A, B pre-activations). */
#define MOK_FLAG_SAVE_FOR_BACKWARD 0x1u
/* Router variants, for the DeepSeek-V3-type models the pages name as the
 * target ([fluid], section "Comment MoK tente de gratter des millisecondes
 * partout").  The selection is the same in every variant: the top-k of the
 * raw fp32 logits (value descending, index ascending).  The gates are the
 * chosen experts' affinities a_e:
 *   default                 a = softmax of the E logits;
 *   MOK_FLAG_SIGMOID_GATES  a_e = sigmoid(logit_e);
 *   MOK_FLAG_RENORM_GATES   gate_j = a_j / (a_0 + ... + a_(k-1)), the sum
 *                           over the k chosen experts in slot order (fp32).
 * The backward call must be given the same flags as its forward call; its
 * d(router logits) is the chain rule through the chosen gates and then the
 * affinity (softmax Jacobian, or a (1 - a) for the sigmoid). */
#define MOK_FLAG_SIGMOID_GATES 0x2u
#define MOK_FLAG_RENORM_GATES 0x4u
/* A forward call of 1 <= T <= 32 tokens and T * k <= 4096 pairs (a decode
 * step, where the launches, not the bytes, set the time of routing and
 * sorting) runs the
 * router and the layout step ([kucoin §01]: count each expert's tokens, then
 * place them, one expert's rows together) as one single-workgroup launch; its stage events then cover MOK_STAGE_ROUTER only,
 * and MOK_STAGE_SORT is not run.  Results are bitwise those of the separate
 * router and sort launches, which this flag selects at any size. */
#define MOK_FLAG_SEPARATE_ROUTE_SORT 0x8u
/* Expert products of small BF16 forward calls.  With few rows per expert the
 * two forward products are bound by reading the chosen experts' weights
 * ([kucoin §01]: the expert-grouped GEMM; [fluid], section "Quand la
 * communication devient le vrai problème", names an MoE inference decode
 * kernel as earlier work), so a call of the whole layer with at most 4096
 * token-expert pairs and d, F multiples of 128 may run them as
 * weight-streaming kernels: each weight row read once per 32-row tile straight
 * into registers, the K range split over up to four waves whose fp32 partial
 * sums are added in a fixed order.  Without either flag below they run when
 * T * k <= 4 * (expert_end - expert_begin) (a few rows per expert on
 * average); MOK_FLAG_STREAM_GEMMS selects them for every such call,
 * MOK_FLAG_TILED_GEMMS never (both: MOK_ERR_INVALID_ARG).  The results are
 * deterministic and within the BF16 tolerance of the oracle, but not bitwise
 * those of the tiled kernels (another summation order).  An MXFP8 forward
 * that saves nothing for backward (d a multiple of 256) follows the same
 * rule, with up to 8 * (expert_end - expert_begin) pairs by default, with
 * MXFP8 weight-streaming kernels (E4M3 codes and their scales read once per
 * 32-row tile; H quantised along F in UP's epilogue as in the tiled path);
 * within the MXFP8 tolerance of the oracle. */
#define MOK_FLAG_TILED_GEMMS 0x10u
#define MOK_FLAG_STREAM_GEMMS 0x20u
/* MXFP8 weight gradients (with MOK_PREC_MXFP8 and MOK_FLAG_SAVE_FOR_BACKWARD
 * only; the pages report the layer's backward time in MXFP8, [kucoin §03],
 * with no recipe): mok_moe_backward_mxfp8 then also computes dW2, dW1 and
 * dW3 on the scaled MFMA.  Their contraction runs over an expert's rows, so
 * each operand (dY, H = silu(A) * B before its quantisation, dA, dB and the x
 * rows) is quantised along the rows: per column, blocks of 32 consecutive
 * rows of the expert's segment from its first row in placement order, the
 * last block taking its scale from the rows it has; then
 *   dW2_e = Qr(dY_e)^T Qr(H_e),  dW1_e = Qr(dA_e)^T Qr(X_e),
 *   dW3_e = Qr(dB_e)^T Qr(X_e),  fp32 results.
 * Requires d to be a multiple of 256 (MOK_ERR_INVALID_ARG otherwise).
 * Without the flag the MXFP8 backward takes these products in bf16.  The
 * workspace of such a configuration holds the transposed codes (see
 * mok_workspace_layout.wq). */
#define MOK_FLAG_MXFP8_WGRAD 0x40u

typedef struct mok_moe_config {
  int32_t T;                 /* tokens in this call (>= 0)                      */
  int32_t d;                 /* hidden size                                     */
  int32_t E;                 /* experts routed over (1..1024)                   */
  int32_t ffn;               /* expert FFN width F                              */
  int32_t expert_begin;      /* first local expert                              */
  int32_t expert_end;        /* one past the last local expert                  */
  int32_t precision;         /* mok_precision                                   */
  int32_t minibatch_rows;    /* R: rows of the expert-sorted buffer processed
                                per minibatch; 0 = the whole layer at once.
                                The pages' minibatch trade-off ([kucoin §02]).
                                R > 0 (BF16 only) runs the ring pipeline: one
                                launch per minibatch m copies minibatch m+1
                                into its ring slot while UP runs on m and DOWN
                                on m-1.  Results are bitwise those of R = 0.
                                T*d*2 < 2^31 (the copies and the backward's
                                gathered x rows use 32-bit offsets).
                                How the workgroups share the copying and the
                                computing: see mover_cus.                    */
  int64_t ring_bytes;        /* fixed ring token buffer for dispatched rows
                                ([fluid], [kucoin §02] "macrobatch"), used
                                with R > 0: floor(ring_bytes / (2 d R)) slots
                                of R rows, at least 2 (else
                                MOK_ERR_WORKSPACE); must be 0 when R = 0.       */
  uint32_t flags;            /* MOK_FLAG_*                                      */
  int32_t mover_cus;         /* R > 0: compute units (one workgroup each) that
                                do only the row copies of each ring launch,
                                the others only the UP and DOWN tiles (the
                                pages' explicit split of SMs between moving
                                tokens and expert compute, [kucoin §02]);
                                0 = no split: all 256 workgroups take every
                                task (the copies of minibatch m+1, 16 rows
                                each, the UP tiles of m and the DOWN tiles of
                                m-1) from eight per-XCD runs through device
                                counters.  0..255; must be 0 when R = 0.
                                Results are the same bits for every value. */
  void* const* stage_events; /* NULL, or 2*MOK_NUM_STAGES hipEvent_t handles
                                (created by the caller): the call records
                                events[2s] on its stream before stage s and
                                events[2s+1] after it, for every stage it runs,
                                so the caller can time each kernel.            */
} mok_moe_config;

/* Stages of one forward or backward call, in launch order. */
typedef enum {
  MOK_STAGE_ROUTER = 0,      /* softmax + top-k                                 */
  MOK_STAGE_SORT = 1,        /* counting sort (histogram, scan, placement)      */
  MOK_STAGE_DISPATCH = 2,    /* gather rows (+ MXFP8 quantise)                  */
  MOK_STAGE_GEMM_UP = 3,     /* H = silu(X W1^T) * (X W3^T)                     */
  MOK_STAGE_GEMM_DOWN = 4,   /* Y = H W2^T                                      */
  MOK_STAGE_COMBINE = 5,     /* out = sum_j gate * Y                            */
  MOK_STAGE_BWD_GATE = 6,    /* dgate, drouter_logits, dY = gate * dout         */
  MOK_STAGE_GEMM_DH = 7,     /* dA, dB from dY W2                               */
  MOK_STAGE_GEMM_DX = 8,     /* dX_perm = dA W1 + dB W3                         */
  MOK_STAGE_REDUCE_DX = 9,   /* dx = sum_j dX_perm                              */
  MOK_STAGE_GEMM_DW2 = 10,   /* dW2 = dY^T H                                    */
  MOK_STAGE_REGATHER = 11,   /* gather X rows again for dW1, dW3                */
  MOK_STAGE_GEMM_DW13 = 12,  /* dW1 = dA^T X, dW3 = dB^T X                      */
  MOK_NUM_STAGES = 13
} mok_stage;

/* Byte offsets of the arrays inside the opaque `saved` buffer (from its base,
 * each 256-byte aligned).  P_max = T*k rows are reserved; only the first P
 * (= expert_offsets[E]) are meaningful. */
typedef struct mok_saved_layout {
  size_t lse;                /* float  [T]        log-sum-exp of each logit row */
  size_t topk_idx;           /* int32  [T*k]                                    */
  size_t topk_gate;          /* float  [T*k]                                    */
  size_t offsets;            /* int32  [E+1]                                    */
  size_t row_of_pair;        /* int32  [T*k]      -1 where the expert is remote */
  size_t pair_of_row;        /* int32  [P_max]                                  */
  size_t A;                  /* act    [P_max, F] x W1^T (pre-activation)       */
  size_t B;                  /* act    [P_max, F] x W3^T                        */
  size_t H;                  /* act    [P_max, F] silu(A) * B                   */
  size_t Y;                  /* act    [P_max, d] expert output, unscaled       */
  size_t total;
} mok_saved_layout;

/* Sizes of the caller-provided buffers for this configuration.
 *   workspace_bytes: scratch for one forward or backward call (dispatch ring
 *                    or full dispatch buffer, counting-sort tables, backward
 *                    intermediates).  Not preserved between calls.
 *   saved_bytes:     what forward writes and backward reads (see
 *                    mok_saved_layout).
 * Returns MOK_ERR_INVALID_ARG for invalid shapes. */
mok_status mok_moe_workspace_query(const mok_moe_config* cfg, int32_t k,
                                   size_t* workspace_bytes, size_t* saved_bytes);

/* Offsets of the arrays inside `saved` (host-only computation). */
mok_status mok_moe_saved_layout(const mok_moe_config* cfg, int32_t k, mok_saved_layout* out);

/* Byte offsets inside the `workspace` buffer (from its base, each 256-byte
 * aligned; host-only computation).  Its contents are scratch of one call,
 * except for the status word, which the caller may read after the call.
 *
 *   status    two int32 words.  Every forward and backward call clears them
 *             when it starts (its first kernel, on the call's stream).  A
 *             device-side check that fails stores MOK_ERR_DEVICE in word 0
 *             and ORs its bit into word 1; the call's outputs are then not
 *             meaningful.  The checks:
 *               MOK_CHECK_LOGITS  a router logit row holds NaN or +-Inf (the
 *                                 chosen indices still lie in [0, E): a NaN
 *                                 ranks below every number);
 *               MOK_CHECK_INDEX   an entry of the row maps or of topk_idx that
 *                                 a backward call reads from `saved` lies
 *                                 outside its range (the slot is then treated
 *                                 as remote, so no access leaves a buffer);
 *             The library never synchronises: read the words (8 bytes at this
 *             offset) once the stream has passed the call, e.g. with a device
 *             to host copy at the caller's own synchronisation point.
 *   xp        the dispatch buffer, or the ring of minibatch slots, then (MXFP8
 *             backward) the dY codes [P_max, d]; MXFP4: E2M1 codes
 *             [xp_rows, d/2] bytes, element 2i in the low nibble of byte i;
 *   xp_scale  MXFP8, MXFP4: its E8M0 scales in pair planes [d/64, xp_rows, 2];
 *   xp_rows   rows held by xp (P_max = T*k, or the ring's rows);
 *   hq, hq_scale  MXFP8 and MXFP4: the H rows [P_max, F] as the first product
 *             quantises them along F for the second (E4M3 bytes, or E2M1
 *             codes two per byte, [P_max, F/2]), and their E8M0 scales in
 *             pair planes [F/64, P_max, 2] (an MXFP8 backward then reuses
 *             both for [dA | dB], 2F wide); nothing otherwise;
 *   dy, dab, dxp  backward row buffers dY [P_max, d], [dA | dB] [P_max, 2F],
 *             dX_perm [P_max, d] (bf16; absent from an MXFP8 forward-only
 *             configuration; no dY rows with MOK_FLAG_MXFP8_WGRAD, whose
 *             weight gradients form dY again from dout and the gates);
 *   wq, wq_scale, k_pad  with MOK_FLAG_MXFP8_WGRAD: the row-quantised
 *             operands of the weight gradients, transposed: E4M3 codes of dY
 *             (d rows), H (F rows), [dA | dB] (2F rows) and x (d rows), each
 *             row k_pad = 128 (floor(T k / 128) + E_loc) bytes long, local
 *             expert e's rows at columns [128 p_e, 128 p_(e+1)) with p the
 *             prefix of ceil(rows / 128) over the local experts (zero codes
 *             past its rows); then their E8M0 scales, for each matrix in pair
 *             planes [k_pad / 64, rows, 2] (byte (j, c, b) = scale of block
 *             2 j + b of row c).  k_pad = 0 and no bytes otherwise;
 *   total     workspace_bytes. */
#define MOK_CHECK_LOGITS 0x1
#define MOK_CHECK_INDEX 0x2
typedef struct mok_workspace_layout {
  size_t status;
  size_t xp;
  size_t xp_scale;
  int64_t xp_rows;
  size_t hq;
  size_t hq_scale;
  size_t dy;
  size_t dab;
  size_t dxp;
  size_t wq;
  size_t wq_scale;
  int64_t k_pad;
  size_t total;
} mok_workspace_layout;

mok_status mok_moe_workspace_layout(const mok_moe_config* cfg, int32_t k, mok_workspace_layout* out);

/*
 * Forward pass of the MoE layer ([kucoin §01-§03]: router, layout, dispatch,
 * grouped expert GEMMs, combine and the final weighted sum).
 *
 *   x              act   [T, d]
 *   router_logits  float [T, E]    finite values
 *   W1, W3         [E_loc, F, d]   gate / up projections (act type; E4M3
 *                                  bytes for MXFP8; for MXFP4 E2M1 codes,
 *                                  two per byte: [E_loc, F, d/2] bytes)
 *   W2             [E_loc, d, F]   down projection (act type; E4M3 for MXFP8;
 *                                  E2M1 [E_loc, d, F/2] bytes for MXFP4)
 *   w_scales       MXFP8 and MXFP4 only, else NULL: E8M0 bytes,
 *                  concatenated: those of W1 as a [E_loc*F, d] matrix, then of
 *                  W3 (same), then of W2 as a [E_loc*d, F] matrix, each in the
 *                  pair-plane layout that mok_quantize_mxfp8 (and
 *                  mok_quantize_mxfp4) writes
 *   out            act   [T, d]    sum_j gate[t,j] * y(t,j), j ascending, in
 *                                  fp32, rounded once; rows of tokens with no
 *                                  local pair are 0
 *   topk_idx       int32 [T, k]    experts by (logit desc, index asc)
 *   topk_gate      float [T, k]    softmax over all E at those experts (not
 *                                  renormalised)
 *   expert_counts  int32 [E]       local pairs per expert (0 for remote)
 *   expert_offsets int32 [E+1]     exclusive prefix sum of expert_counts
 *   saved          mok_saved_layout.total bytes
 *   workspace      workspace_bytes bytes
 * Alignment: every pointer 16-byte aligned.  Constraints: 1 <= k <= E <= 1024,
 * d and F multiples of 64 (bf16), 128 (MXFP8), 256 (MXFP4) or 16 (fp32),
 * T*k < 2^31.
 * MXFP4 (an MXFP4 analogue of the NVFP4 kernels tried before the
 * megakernel, [fluid «Quand la communication devient le vrai problème»]):
 * the MXFP8 forward with E2M1 elements (OCP Microscaling v1.0 MXFP4: scale
 * 2^(floor(log2 amax) - 2) per 32 values, elements rounded to nearest even,
 * saturating at 6): x rows quantised by the dispatch, H along F by the first
 * product's epilogue, the weights by mok_quantize_mxfp4.  Forward only:
 * MOK_FLAG_SAVE_FOR_BACKWARD (and a ring) give MOK_ERR_UNSUPPORTED.
 */
mok_status mok_moe_forward(const void* x, const float* router_logits,
                           const void* W1, const void* W3, const void* W2, int32_t k,
                           const mok_moe_config* cfg, const uint8_t* w_scales,
                           void* out, int32_t* topk_idx, float* topk_gate,
                           int32_t* expert_counts, int32_t* expert_offsets,
                           void* saved, void* workspace, void* stream);

/*
 * Forward for callers that cannot allocate device memory: code being captured
 * into a HIP graph, tight serving loops, harnesses that forbid allocation.  The
 * same computation and arguments as mok_moe_forward without `workspace`: its
 * scratch (the status words and the counting sort's chunk tables) lives in a
 * static device array of the library, 4 MiB per GPU, held until the process
 * ends.  Nothing is allocated or freed by the call.
 *   Supports the bf16 whole layer (MOK_PREC_BF16, minibatch_rows = 0, x below
 *   2 GiB) with or without MOK_FLAG_SAVE_FOR_BACKWARD and the router variant
 *   flags; other configurations return MOK_ERR_UNSUPPORTED.  The scratch
 *   needed is about 8 * E * ceil(T*k / 512) bytes; beyond 4 MiB the call
 *   returns MOK_ERR_WORKSPACE (at E 128, up to T*k of about 2 million pairs).
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (other streams, other threads) race and must be serialised by the
 *   caller.  The array is taken on the device current when the call is made,
 *   which must be the device of `stream`.  The device status words are kept
 *   in the array and are not readable by the caller.
 * `saved` is still the caller's (as for mok_moe_forward; a later
 * mok_moe_backward needs a workspace of its own).
 */
mok_status mok_moe_forward_noalloc(const void* x, const float* router_logits,
                                   const void* W1, const void* W3, const void* W2, int32_t k,
                                   const mok_moe_config* cfg, void* out, int32_t* topk_idx,
                                   float* topk_gate, int32_t* expert_counts, int32_t* expert_offsets,
                                   void* saved, void* stream);

/*
 * Backward pass: gradients of L = sum(out * dout), mirroring the forward
 * ([kucoin §01]: two more communication steps in the reverse direction;
 * [kucoin §02]: reverse-combine, then reverse-dispatch).  Requires a forward
 * call with MOK_FLAG_SAVE_FOR_BACKWARD on the same inputs and `saved`.
 *
 *   dout           act   [T, d]
 *   dx             act   [T, d]    expert path only: sum_j of the pair
 *                                  gradients, j ascending, fp32, rounded once
 *   dW1, dW3       float [E_loc, F, d]   overwritten (not accumulated)
 *   dW2            float [E_loc, d, F]   overwritten
 *   dgate          float [T, k]    <dout_t, y(t,j)>; 0 for remote pairs
 *   drouter_logits float [T, E]    p * (G - <p, G>), G = dgate scattered
 * BF16 and FP32 precisions (MXFP8: mok_moe_backward_mxfp8; this call then
 * returns MOK_ERR_UNSUPPORTED).
 */
mok_status mok_moe_backward(const void* dout, const void* x, const float* router_logits,
                            const void* W1, const void* W3, const void* W2, int32_t k,
                            const mok_moe_config* cfg, const void* saved,
                            void* dx, float* dW1, float* dW3, float* dW2,
                            float* dgate, float* drouter_logits,
                            void* workspace, void* stream);

/*
 * MXFP8 backward ([kucoin §03] reports the layer's backward time in MXFP8;
 * the pages give no recipe, so this is the reading taken): the same outputs
 * as mok_moe_backward, after an MXFP8 forward call with
 * MOK_FLAG_SAVE_FOR_BACKWARD (which then also saves A, B and H before its
 * quantisation as bf16).  The two products that lead to dx run on scaled
 * MFMA with each operand quantised along the axis it contracts:
 *   dH = Q_d(dY) Q_d(W2^T)^T, then dA, dB by the SwiGLU backward,
 *   dX_perm = Q_F(dA) Q_F(W1^T)^T + Q_F(dB) Q_F(W3^T)^T,
 * dY (= gate * dout) quantised inside the reverse-combine and [dA | dB]
 * inside the dH epilogue.  The weight gradients are bf16 products of the
 * unquantised operands (dY, H, dA, dB and x rows), fp32 results.
 *   wt_e4m3, wt_e8m0  the transposed weights from
 *                     mok_quantize_mxfp8_backward_weights
 *   dout, x            bf16 [T, d]; other arguments as in mok_moe_backward
 * Errors: MOK_ERR_INVALID_ARG unless cfg->precision is MOK_PREC_MXFP8 and the
 * save flag is set, plus mok_moe_backward's checks.
 */
mok_status mok_moe_backward_mxfp8(const void* dout, const void* x, const float* router_logits, int32_t k,
                                  const mok_moe_config* cfg, const uint8_t* wt_e4m3,
                                  const uint8_t* wt_e8m0, const void* saved, void* dx, float* dW1,
                                  float* dW3, float* dW2, float* dgate, float* drouter_logits,
                                  void* workspace, void* stream);

/*
 * Transposed MXFP8 copies of the expert weights for mok_moe_backward_mxfp8
 * (quantisation rule of mok_quantize_mxfp8; once per weight update, outside
 * the layer call, like the forward's weights):
 *   W1, W3   bf16 [E_loc, F, d];  W2  bf16 [E_loc, d, F]
 *   wt_e4m3  3 * E_loc * F * d bytes: W2^T as [E_loc, F, d] (each row a
 *            column of W2_e, quantised along d), then [W1^T | W3^T] as
 *            [E_loc, d, 2F] (row i holds column i of W1_e, then of W3_e,
 *            quantised along F)
 *   wt_e8m0  3 * E_loc * F * d / 32 bytes: the scales of W2^T as pair planes
 *            [d/64, E_loc*F, 2], then those of [W1^T | W3^T] as
 *            [2F/64, E_loc*d, 2] (the layout of mok_quantize_mxfp8)
 * Errors: MOK_ERR_INVALID_ARG for a null or misaligned pointer, E_loc < 1,
 * d or F not a multiple of 128, or a scale array of 2^32 bytes or more.
 */
mok_status mok_quantize_mxfp8_backward_weights(const void* W1, const void* W3, const void* W2, int32_t E_loc,
                                               int32_t d, int32_t F, uint8_t* wt_e4m3, uint8_t* wt_e8m0,
                                               void* stream);

/*
 * MXFP8 quantisation of a bf16 matrix along its rows ([kucoin §02]: MXFP8
 * activation quantisation; the rule is OCP Microscaling v1.0): per block of
 * 32 consecutive elements of a row, scale X = 2^(floor(log2 amax) - 8) stored
 * as an E8M0 byte (exponent + 127, clamped to [0, 254]; an all-zero block
 * stores 0), elements E4M3(v / X) rounded to nearest even, saturating at 448.
 *   src_bf16  [rows, K]      K a multiple of 64, rows * K / 32 < 2^32
 *   dst_e4m3  [rows, K]      bytes
 *   dst_e8m0  rows * K / 32 bytes in pair planes: the scale of block b of
 *             row r (elements 32 b .. 32 b + 31) at byte
 *             (b / 2) * 2 rows + 2 r + (b % 2), i.e. a [K/64, rows, 2] array,
 *             so that the scales of consecutive rows for one 64-wide K step
 *             are adjacent (the GEMMs copy them 128 contiguous bytes at a
 *             time; the layer's own activation scales use the same layout)
 * Used for the weights (once per weight update, outside the layer call); the
 * layer quantises activations itself, inside its dispatch and SwiGLU steps.
 * Errors: MOK_ERR_INVALID_ARG for a null or misaligned pointer, K not a
 * multiple of 64, or a scale array of 2^32 bytes or more.
 */
mok_status mok_quantize_mxfp8(const void* src_bf16, int64_t rows, int64_t K,
                              uint8_t* dst_e4m3, uint8_t* dst_e8m0, void* stream);

/*
 * MXFP4 quantisation of a bf16 matrix along its rows, for the weights of an
 * MXFP4 forward (OCP Microscaling v1.0 MXFP4; the analogue of the NVFP4
 * attempt of [fluid «Quand la communication devient le vrai problème»]): per
 * block of 32 consecutive elements of a row, scale X = 2^(floor(log2 amax) -
 * 2) stored as an E8M0 byte (exponent + 127, clamped to [0, 254]; an all-zero
 * block stores 0), elements E2M1(v / X) (S.EE.M, bias 1: magnitudes 0, 0.5,
 * 1, 1.5, 2, 3, 4, 6) rounded to nearest even, saturating at 6, the sign of
 * zero kept.
 *   src_bf16  [rows, K]      K a multiple of 64, rows * K / 32 < 2^32
 *   dst_e2m1  [rows, K / 2]  bytes; element 2i of a row in the low nibble of
 *             byte i, element 2i + 1 in the high nibble
 *   dst_e8m0  rows * K / 32 bytes in the pair planes of mok_quantize_mxfp8
 * Errors: MOK_ERR_INVALID_ARG for a null or misaligned pointer, K not a
 * multiple of 64, or a scale array of 2^32 bytes or more.
 */
mok_status mok_quantize_mxfp4(const void* src_bf16, int64_t rows, int64_t K,
                              uint8_t* dst_e2m1, uint8_t* dst_e8m0, void* stream);

/*
 * Router GEMM: the scores the router step consumes ([kucoin §01]: the router
 * scores each token against every expert before the top-k choice; here a
 * score is the dot product of the token with the expert's router vector):
 *   logits[t, e] = sum_i x[t, i] * Wr[e, i]
 *   x       bf16  [T, d]
 *   Wr      bf16  [E, d]   one row per expert
 *   logits  float [T, E]   overwritten; products exact, fp32 accumulation in
 *                          an order fixed by (T, d, E)
 * d a multiple of 64 and at most 65536, 1 <= E <= 1024, 0 <= T <= 2^24;
 * x and Wr 16-byte aligned.  The result feeds mok_moe_forward's
 * router_logits.
 * Errors: MOK_ERR_INVALID_ARG for a null or misaligned pointer or a shape
 * outside these bounds; MOK_ERR_HIP for a failed launch.
 */
mok_status mok_router_logits(const void* x, const void* Wr, int32_t T, int32_t d, int32_t E,
                             float* logits, void* stream);

/*
 * Gradients through mok_router_logits of L = sum(logits * dlogits):
 *   dlogits float [T, E]   e.g. mok_moe_backward's drouter_logits
 *   dx      float [T, d] = dlogits . Wr     (overwritten)
 *   dWr     float [E, d] = dlogits^T . x    (overwritten; T = 0 gives 0)
 * dlogits enters the bf16 matrix cores as a bf16 value plus a bf16 residual
 * (relative residual below 2^-17); x and Wr are exact.  dWr sums the tokens
 * in slices whose partial products are kept in dx's memory before dx is
 * written, then adds the slices in ascending order: dx must not overlap
 * dWr, x, Wr or dlogits.  Shapes and pointers as for mok_router_logits;
 * dx and dWr 16-byte aligned.
 * Errors: MOK_ERR_INVALID_ARG, MOK_ERR_HIP as for mok_router_logits.
 */
mok_status mok_router_logits_backward(const void* x, const void* Wr, const float* dlogits, int32_t T,
                                      int32_t d, int32_t E, float* dx, float* dWr, void* stream);

/*
 * Forward pass with the router GEMM in front: x . Wr^T -> softmax / top-k ->
 * the layer ([kucoin §01]: the router scores every token against every
 * expert and picks its experts; the router GEMM fused into the router step,
 * so the [T, E] logits are not read back).  Equivalent, bit for bit in every
 * output, to mok_router_logits(x, Wr, ..., router_logits) followed by
 * mok_moe_forward(x, router_logits, ...).
 *   Wr             bf16  [E, d]   router vectors, one row per expert
 *   router_logits  float [T, E]   output (the backward reads them)
 *   all other arguments as mok_moe_forward
 * For E <= 128 one kernel computes a tile of 32 tokens' logits, writes them,
 * and routes those tokens from the copy it holds in LDS; for E > 128 the
 * router GEMM and the router step are two launches; calls of at most 32
 * tokens run the router GEMM and then the one-launch router and sort.
 * Constraints: those of mok_moe_forward and of mok_router_logits (d <= 65536);
 * bf16 activations (MOK_PREC_BF16, MOK_PREC_MXFP8, MOK_PREC_MXFP4).
 * Errors: MOK_ERR_INVALID_ARG for MOK_PREC_F32, a null or misaligned Wr or
 * router_logits, or any error of mok_moe_forward.
 */
mok_status mok_moe_forward_router(const void* x, const void* Wr, const void* W1, const void* W3, const void* W2,
                                  int32_t k, const mok_moe_config* cfg, const uint8_t* w_scales,
                                  float* router_logits, void* out, int32_t* topk_idx, float* topk_gate,
                                  int32_t* expert_counts, int32_t* expert_offsets, void* saved, void* workspace,
                                  void* stream);

/* Static, human-readable name of a status code. */
const char* mok_status_string(mok_status s);

/* Library version as major*10000 + minor*100 + patch. */
int32_t mok_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOK_H_ */
