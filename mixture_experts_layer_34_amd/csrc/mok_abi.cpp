// C ABI of the MoE layer (include/mok.h): argument validation, buffer layouts
// and the launch sequence of one layer call.  Everything here runs on the
// host before any launch; a call enqueues its kernels on the caller's stream
// and returns without synchronising or allocating (the pages' layer has no
// host round trip inside it: laura-martel.com post on Mixture-of-Kittens,
// section "Ce qu'il fait réellement"; fluidifia.com, "Cursor ouvre MoK, un
// mégakernel qui accélère l'entraînement MoE", section "Quand la
// communication devient le vrai problème").
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "../../include/mok.h"
#include "mok_internal.h"
#include "router_gemm.h"

using namespace mok;

typedef uint16_t bf16_t_;  // bf16 storage (host side)

namespace {

enum { KIND_UP = 0, KIND_DOWN = 1, KIND_DH = 2, KIND_DX = 3, KIND_DW2 = 4, KIND_DW13 = 5 };

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t act_size(const mok_moe_config& c) { return c.precision == MOK_PREC_F32 ? 4 : 2; }

mok_status validate_config(const mok_moe_config* cfg, int32_t k) {
  if (!cfg) return MOK_ERR_INVALID_ARG;
  const mok_moe_config& c = *cfg;
  if (c.T < 0 || c.d <= 0 || c.ffn <= 0 || c.E < 1 || c.E > 1024) return MOK_ERR_INVALID_ARG;
  if (k < 1 || k > c.E) return MOK_ERR_INVALID_ARG;
  if (c.expert_begin < 0 || c.expert_end <= c.expert_begin || c.expert_end > c.E) return MOK_ERR_INVALID_ARG;
  if (c.precision != MOK_PREC_F32 && c.precision != MOK_PREC_BF16 && c.precision != MOK_PREC_MXFP8 &&
      c.precision != MOK_PREC_MXFP4)
    return MOK_ERR_INVALID_ARG;
  // bf16: K steps of 64; MXFP8: K steps of 128 bytes (and whole MX blocks);
  // MXFP4: 128 bytes = 256 values; fp32: 16
  const int mult = c.precision == MOK_PREC_F32
                       ? 16
                       : (c.precision == MOK_PREC_MXFP8 ? 128 : (c.precision == MOK_PREC_MXFP4 ? 256 : 64));
  if (c.d % mult || c.ffn % mult) return MOK_ERR_INVALID_ARG;
  if ((int64_t)c.T * k >= (int64_t(1) << 31)) return MOK_ERR_INVALID_ARG;
  if ((int64_t)c.T * k * (int64_t)(c.d > 2 * c.ffn ? c.d : 2 * c.ffn) >= (int64_t(1) << 40))
    return MOK_ERR_INVALID_ARG;
  if (c.minibatch_rows < 0 || c.ring_bytes < 0) return MOK_ERR_INVALID_ARG;
  if (c.mover_cus < 0 || c.mover_cus > 255 || (c.mover_cus > 0 && c.minibatch_rows == 0)) return MOK_ERR_INVALID_ARG;
  if (c.flags & ~(MOK_FLAG_SAVE_FOR_BACKWARD | MOK_FLAG_SIGMOID_GATES | MOK_FLAG_RENORM_GATES |
                  MOK_FLAG_SEPARATE_ROUTE_SORT | MOK_FLAG_TILED_GEMMS | MOK_FLAG_STREAM_GEMMS |
                  MOK_FLAG_MXFP8_WGRAD))
    return MOK_ERR_INVALID_ARG;
  if (c.flags & MOK_FLAG_MXFP8_WGRAD) {
    // MXFP8 training only; the GEMMs address 256 rows of the transposed
    // operands (k_pad bytes each) through one 32-bit buffer range
    if (c.precision != MOK_PREC_MXFP8 || !(c.flags & MOK_FLAG_SAVE_FOR_BACKWARD)) return MOK_ERR_INVALID_ARG;
    if (c.d % 256) return MOK_ERR_INVALID_ARG;  // dW2 rows come in tiles of 256 (2F is a multiple of 256)
    const int64_t kp = 128 * ((int64_t)c.T * k / 128 + (c.expert_end - c.expert_begin));
    if (kp * 256 >= (int64_t(1) << 32)) return MOK_ERR_INVALID_ARG;
  }
  if ((c.flags & MOK_FLAG_TILED_GEMMS) && (c.flags & MOK_FLAG_STREAM_GEMMS)) return MOK_ERR_INVALID_ARG;
  // MXFP4 is a forward (inference) precision: nothing is saved for a backward
  if (c.precision == MOK_PREC_MXFP4 && (c.flags & MOK_FLAG_SAVE_FOR_BACKWARD)) return MOK_ERR_UNSUPPORTED;
  if (c.precision == MOK_PREC_MXFP8 || c.precision == MOK_PREC_MXFP4) {
    // every E8M0 scale array (x and H rows, each weight matrix) fits a 32-bit buffer range
    const int64_t Tk = (int64_t)c.T * k, kmax = c.d > c.ffn ? c.d : c.ffn;
    const int64_t E_loc = c.expert_end - c.expert_begin;
    if (Tk * (kmax / 32) >= (int64_t(1) << 32) || E_loc * c.ffn * (int64_t)(c.d / 32) >= (int64_t(1) << 32))
      return MOK_ERR_INVALID_ARG;
    // the backward's [dA | dB] scales (2F per row)
    if ((c.flags & MOK_FLAG_SAVE_FOR_BACKWARD) && Tk * (2 * (int64_t)c.ffn / 32) >= (int64_t(1) << 32))
      return MOK_ERR_INVALID_ARG;
  }
  if (c.ring_bytes > 0 && c.minibatch_rows == 0) return MOK_ERR_INVALID_ARG;  // a ring needs a minibatch size
  if (c.minibatch_rows > 0) {
    if (c.precision != MOK_PREC_BF16) return MOK_ERR_UNSUPPORTED;
    // the ring's row copies and the backward's gathered x rows address x
    // through 32-bit buffer offsets
    if ((int64_t)c.T * c.d * 2 >= (int64_t(1) << 31)) return MOK_ERR_INVALID_ARG;
    // two slots at least: minibatch m+1 is copied while m is read
    if (c.ring_bytes < 2 * (int64_t)c.minibatch_rows * c.d * 2) return MOK_ERR_WORKSPACE;
  }
  return MOK_OK;
}

// Ring slots of R rows each (minibatch mode), never more than minibatches.
int ring_slots(const mok_moe_config& c, int32_t k) {
  const int64_t R = c.minibatch_rows, Tk = (int64_t)c.T * k;
  const int64_t M = (Tk + R - 1) / R;
  int64_t S = c.ring_bytes / ((int64_t)c.d * 2) / R;
  if (S > M) S = M;
  return (int)(S < 1 ? 1 : S);
}

// Public arrays (mok_saved_layout) plus two internal ones: the per-expert
// row-tile prefix and the experts ranked by row count.
struct SavedLayout {
  mok_saved_layout pub;
  size_t tile_prefix, expert_order;
};

void saved_layout(const mok_moe_config& c, int32_t k, mok_saved_layout* s, size_t* tile_prefix_off,
                  size_t* expert_order_off) {
  const size_t Tk = (size_t)c.T * k, A = act_size(c);
  const size_t E_loc = (size_t)(c.expert_end - c.expert_begin);
  size_t o = 0;
  s->lse = o;          o = align256(o + (size_t)c.T * 4);
  s->topk_idx = o;     o = align256(o + Tk * 4);
  s->topk_gate = o;    o = align256(o + Tk * 4);
  s->offsets = o;      o = align256(o + ((size_t)c.E + 1) * 4);
  *tile_prefix_off = o; o = align256(o + (size_t)kNumTileBM * (E_loc + 1) * 4);
  *expert_order_off = o; o = align256(o + (size_t)(E_loc + 1) * 16);
  s->row_of_pair = o;  o = align256(o + Tk * 4);
  s->pair_of_row = o;  o = align256(o + Tk * 4);
  s->A = o;            o = align256(o + Tk * c.ffn * A);
  s->B = o;            o = align256(o + Tk * c.ffn * A);
  s->H = o;            o = align256(o + Tk * c.ffn * A);
  s->Y = o;            o = align256(o + Tk * c.d * A);
  s->total = o;
}

template <typename T> T* at(void* base, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(base) + off); }
template <typename T> const T* at(const void* base, size_t off) {
  return reinterpret_cast<const T*>(static_cast<const char*>(base) + off);
}

void workspace_layout(const mok_moe_config& c, int32_t k, WorkspaceLayout* w) {
  const size_t Tk = (size_t)c.T * k, A = act_size(c);
  const int64_t nchunks = ((int64_t)Tk + kSortChunk - 1) / kSortChunk;
  const size_t E_loc = (size_t)(c.expert_end - c.expert_begin);
  const bool mx = c.precision == MOK_PREC_MXFP8 || c.precision == MOK_PREC_MXFP4;
  const size_t epb = c.precision == MOK_PREC_MXFP4 ? 2 : 1;  // MX codes per byte
  // MXFP8 training: the backward's bf16 buffers as in bf16 mode; its MXFP8 dY
  // reuses the dispatch buffer and [dA | dB] the (then twice as wide) H buffer
  const bool mxb = mx && (c.flags & MOK_FLAG_SAVE_FOR_BACKWARD);
  const size_t hq_cols = (size_t)c.ffn * (mxb ? 2 : 1);
  w->nchunks = (int)nchunks;
  w->xp_rows = c.minibatch_rows > 0 ? (int64_t)ring_slots(c, k) * c.minibatch_rows : (int64_t)Tk;
  size_t o = 0;
  w->status = o;        o = align256(o + 256);
  w->chunk_counts = o;  o = align256(o + (size_t)nchunks * c.E * 4);
  w->chunk_base = o;    o = align256(o + (size_t)nchunks * c.E * 4);
  w->tile_prefix = o;   o = align256(o + (size_t)kNumTileBM * (E_loc + 1) * 4);
  w->xp = o;            o = align256(o + (mx ? (size_t)w->xp_rows * c.d / epb : (size_t)w->xp_rows * c.d * A));
  w->xp_scale = o;      o = align256(o + (mx ? (size_t)w->xp_rows * (c.d / 32) : 0));
  w->hq = o;            o = align256(o + (mx ? Tk * hq_cols / epb : 0));
  w->hq_scale = o;      o = align256(o + (mx ? Tk * (hq_cols / 32) : 0));
  // MXFP8 weight gradients form dY again from dout: no bf16 dY rows
  const bool mxw_dy = mxb && (c.flags & MOK_FLAG_MXFP8_WGRAD);
  w->dy = o;            o = align256(o + ((mx && !mxb) || mxw_dy ? 0 : Tk * c.d * A));
  w->dab = o;           o = align256(o + (mx && !mxb ? 0 : Tk * 2 * c.ffn * A));
  w->dxp = o;           o = align256(o + (mx && !mxb ? 0 : Tk * c.d * A));
  w->queue = o;         o = align256(o + 256);
  const bool mxw = mxb && (c.flags & MOK_FLAG_MXFP8_WGRAD);
  const int64_t E_loc_ = c.expert_end - c.expert_begin;
  w->k_pad = mxw ? 128 * ((int64_t)Tk / 128 + E_loc_) : 0;
  const size_t wq_rows = (size_t)(2 * c.d + 3 * c.ffn);
  w->wq = o;            o = align256(o + wq_rows * (size_t)w->k_pad);
  w->wq_scale = o;      o = align256(o + wq_rows * (size_t)w->k_pad / 32);
  w->total = o;
}



hipError_t run_gemm(int prec, int kind, const GroupedGemmArgs& g, hipStream_t s) {
  if (prec == MOK_PREC_F32) return gemm_f32(kind, g, s);
  if (prec == MOK_PREC_MXFP8) return gemm_mxfp8(kind, g, s);
  if (prec == MOK_PREC_MXFP4) return gemm_mxfp4(kind, g, s);
  return gemm_bf16(kind, g, s);
}

// Records the caller's stage events around one stage (no-op without events).
struct StageMark {
  const mok_moe_config& c;
  hipStream_t s;
  int stage;
  StageMark(const mok_moe_config& cfg, hipStream_t st, int sg) : c(cfg), s(st), stage(sg) {
    if (c.stage_events) (void)hipEventRecord((hipEvent_t)c.stage_events[2 * stage], s);
  }
  ~StageMark() {
    if (c.stage_events) (void)hipEventRecord((hipEvent_t)c.stage_events[2 * stage + 1], s);
  }
};

// A stage folded into another kernel still gets its (empty) pair of events,
// so that callers timing every stage find them all recorded.
inline void mark_empty_stage(const mok_moe_config& c, hipStream_t s, int stage) {
  if (c.stage_events) {
    (void)hipEventRecord((hipEvent_t)c.stage_events[2 * stage], s);
    (void)hipEventRecord((hipEvent_t)c.stage_events[2 * stage + 1], s);
  }
}

// BF16 without a ring pulls the dispatched rows straight from x inside the
// GEMM loads (32-bit buffer offsets: x must stay below 2 GB).
inline bool fused_pull(const mok_moe_config& c) {
  return c.precision == MOK_PREC_BF16 && c.minibatch_rows == 0 && (int64_t)c.T * c.d * 2 < (int64_t(1) << 31);
}

// The forward's UP and DOWN run the weight-streaming kernels: bf16 with pull
// dispatch, at most kStreamMaxPairs token-expert pairs, K dimensions in whole
// 128-element chunks; then MOK_FLAG_STREAM_GEMMS selects them, and without
// either GEMM flag they run while the call has at most four rows per local
// expert on average (each 32-row tile reads its expert's weights again, so
// with more rows the tiled kernels win: same-box at d 4096, E 128, k 8,
// F 1536, 725 / 742 us at T 64 against 968 / 917 us at T 128, streaming /
// tiled).
constexpr int64_t kStreamMaxPairs = 4096;
constexpr int64_t kStreamAutoRowsPerExpert = 4;
inline bool streaming_gemms(const mok_moe_config& c, int32_t k) {
  const int64_t P = (int64_t)c.T * k, E_loc = c.expert_end - c.expert_begin;
  if (!fused_pull(c) || (c.flags & MOK_FLAG_TILED_GEMMS) || P > kStreamMaxPairs || stream_ksplit(c.d) == 0 ||
      stream_ksplit(c.ffn) == 0)
    return false;
  return (c.flags & MOK_FLAG_STREAM_GEMMS) || P <= kStreamAutoRowsPerExpert * E_loc;
}
// The same choice for an MXFP8 forward that saves nothing for backward
// (inference), and for every MXFP4 forward: whole layer, d a multiple of 256;
// up to eight rows per local expert on average (MXFP8, same-box at d 4096,
// E 128, k 8, F 1536: 653 / 788 us at T 128, streaming / tiled; 266 / 347 us
// at T 16).
constexpr int64_t kStreamAutoRowsPerExpertMx = 8;
inline bool streaming_gemms_mx(const mok_moe_config& c, int32_t k) {
  const int64_t P = (int64_t)c.T * k, E_loc = c.expert_end - c.expert_begin;
  const bool mx = c.precision == MOK_PREC_MXFP8 || c.precision == MOK_PREC_MXFP4;
  if (!mx || c.minibatch_rows != 0 || (c.flags & MOK_FLAG_SAVE_FOR_BACKWARD) ||
      (c.flags & MOK_FLAG_TILED_GEMMS) || P > kStreamMaxPairs || !stream_mx_ok(c.d, c.ffn))
    return false;
  return (c.flags & MOK_FLAG_STREAM_GEMMS) || P <= kStreamAutoRowsPerExpertMx * E_loc;
}

// The call owns every expert (no remote slots).
inline int all_local(const mok_moe_config& c) { return c.expert_begin == 0 && c.expert_end == c.E; }

// The router variant of a call (kGateSigmoid, kGateRenorm bits).
static int gating_of(const mok_moe_config& c) {
  return ((c.flags & MOK_FLAG_SIGMOID_GATES) ? kGateSigmoid : 0) | ((c.flags & MOK_FLAG_RENORM_GATES) ? kGateRenorm : 0);
}

#define MOK_STAGE(stage, call)                 \
  do {                                         \
    StageMark mark_(c, s, stage);              \
    if ((call) != hipSuccess) return MOK_ERR_HIP; \
  } while (0)

#define MOK_HIP(call)                          \
  do {                                         \
    if ((call) != hipSuccess) return MOK_ERR_HIP; \
  } while (0)

// The forward launch sequence, arguments already checked, with the workspace
// at `workspace` laid out as `wl`.  With Wr, the router logits are first
// computed from x and Wr into router_logits (the router GEMM; for E <= 128
// fused with the router step).
mok_status forward_checked(const void* x, const float* router_logits, const void* W1, const void* W3,
                           const void* W2, int32_t k, const mok_moe_config& c, const uint8_t* w_scales,
                           void* out, int32_t* topk_idx, float* topk_gate, int32_t* expert_counts,
                           int32_t* expert_offsets, void* saved, void* workspace, const WorkspaceLayout& wl,
                           void* stream, const void* Wr = nullptr) {
  const bool mx4 = c.precision == MOK_PREC_MXFP4;
  const bool mx = c.precision == MOK_PREC_MXFP8 || mx4;
  hipStream_t s = (hipStream_t)stream;
  const int T = c.T, E = c.E, d = c.d, F = c.ffn, eb = c.expert_begin, E_loc = c.expert_end - c.expert_begin;
  const int bf16 = c.precision != MOK_PREC_F32;
  mok_saved_layout sl;
  size_t tp_off, eo_off;
  saved_layout(c, k, &sl, &tp_off, &eo_off);

  int32_t* s_idx = at<int32_t>(saved, sl.topk_idx);
  float* s_gate = at<float>(saved, sl.topk_gate);
  float* s_lse = at<float>(saved, sl.lse);
  int32_t* s_off = at<int32_t>(saved, sl.offsets);
  int32_t* s_tp = at<int32_t>(saved, tp_off);
  int32_t* s_order = at<int32_t>(saved, eo_off);
  int32_t* s_rop = at<int32_t>(saved, sl.row_of_pair);
  int32_t* s_por = at<int32_t>(saved, sl.pair_of_row);

  int32_t* status = at<int32_t>(workspace, wl.status);
  const int64_t P_max = (int64_t)T * k;
  float* logits_out = const_cast<float*>(router_logits);  // written only when Wr is given
  if (T >= 1 && T <= kSmallTokens && P_max <= kSmallPairs && !(c.flags & MOK_FLAG_SEPARATE_ROUTE_SORT)) {
    // small call: status reset, router and counting sort in one workgroup
    StageMark mark(c, s, MOK_STAGE_ROUTER);
    if (Wr) MOK_HIP(launch_router_logits(x, Wr, T, d, E, logits_out, s));
    MOK_HIP(launch_route_sort_small(router_logits, T, E, k, gating_of(c), eb, c.expert_end, topk_idx, topk_gate,
                                    s_idx, s_gate, s_lse, expert_counts, expert_offsets, s_off, s_tp, s_order, s_rop,
                                    s_por, status, s));
  } else {
    MOK_HIP(launch_status_reset(status, s));
    if (Wr && E <= kRouterFusedMaxE) {
      MOK_STAGE(MOK_STAGE_ROUTER, launch_router_fused(x, Wr, T, d, E, k, gating_of(c), logits_out, topk_idx,
                                                      topk_gate, s_idx, s_gate, s_lse, status, s));
    } else {
      StageMark mark(c, s, MOK_STAGE_ROUTER);
      if (Wr) MOK_HIP(launch_router_logits(x, Wr, T, d, E, logits_out, s));
      MOK_HIP(launch_router_topk(router_logits, T, E, k, gating_of(c), topk_idx, topk_gate, s_idx, s_gate, s_lse,
                                 status, s));
    }
    MOK_STAGE(MOK_STAGE_SORT, launch_counting_sort(s_idx, T, k, E, eb, c.expert_end, wl.nchunks,
                                                   at<int32_t>(workspace, wl.chunk_counts),
                                                   at<int32_t>(workspace, wl.chunk_base), expert_counts,
                                                   expert_offsets, s_off, s_tp, s_order, s_rop, s_por, s));
  }
  GroupedGemmArgs g{};
  g.offsets = s_off;
  g.tile_prefix = s_tp;
  g.expert_order = s_order;
  g.eb = eb;
  g.E_loc = E_loc;
  g.d = d;
  g.F = F;
  g.P_max = (int64_t)T * k;
  if (mx) {
    uint8_t* xq = at<uint8_t>(workspace, wl.xp);
    uint8_t* xs = at<uint8_t>(workspace, wl.xp_scale);
    MOK_STAGE(MOK_STAGE_DISPATCH, mx4 ? launch_dispatch_gather_mxfp4(x, s_rop, T, k, d, xq, xs, wl.xp_rows, status, s)
                                      : launch_dispatch_gather_mxfp8(x, s_rop, T, k, d, xq, xs, wl.xp_rows, status, s));
    const size_t w13_scales = (size_t)E_loc * F * (d / 32);
    g.A = xq;
    g.a_scale = xs;
    g.B0 = W1;
    g.B1 = W3;
    g.b_scale0 = w_scales;
    g.b_scale1 = w_scales + w13_scales;
    g.out0 = at<uint8_t>(workspace, wl.hq);
    g.out_scale = at<uint8_t>(workspace, wl.hq_scale);
    if (c.flags & MOK_FLAG_SAVE_FOR_BACKWARD) {
      g.save = 1;
      g.save_a = at<void>(saved, sl.A);
      g.save_b = at<void>(saved, sl.B);
      g.out1 = at<void>(saved, sl.H);
    }
    const bool stream_mx = streaming_gemms_mx(c, k);
    auto stream_gemm = mx4 ? gemm_stream_mxfp4 : gemm_stream_mxfp8;
    MOK_STAGE(MOK_STAGE_GEMM_UP, stream_mx ? stream_gemm(KIND_UP, g, s) : run_gemm(c.precision, KIND_UP, g, s));
    GroupedGemmArgs g2 = g;
    g2.save = 0;
    g2.out1 = nullptr;
    g2.A = at<uint8_t>(workspace, wl.hq);
    g2.a_scale = at<uint8_t>(workspace, wl.hq_scale);
    g2.B0 = W2;
    g2.B1 = nullptr;
    g2.b_scale0 = w_scales + 2 * w13_scales;
    g2.b_scale1 = nullptr;
    g2.out0 = at<void>(saved, sl.Y);
    g2.out_scale = nullptr;
    MOK_STAGE(MOK_STAGE_GEMM_DOWN,
              stream_mx ? stream_gemm(KIND_DOWN, g2, s) : run_gemm(c.precision, KIND_DOWN, g2, s));
  } else if (c.minibatch_rows > 0) {
    // Ring-buffer minibatch pipeline ([kucoin §02]: tunable minibatches drawn
    // from a fixed ring token buffer; [fluid «Comment MoK…»]): launch m copies
    // minibatch m+1 into its slot, runs UP on minibatch m and DOWN on m-1.
    const int R = c.minibatch_rows, S = ring_slots(c, k);
    const int M = (int)(((int64_t)T * k + R - 1) / R);
    bf16_t_* ring = at<bf16_t_>(workspace, wl.xp);
    MinibatchStepArgs ms{};
    ms.up = g;
    ms.up.A = ring;
    ms.up.B0 = W1;
    ms.up.B1 = W3;
    ms.up.out0 = at<void>(saved, sl.H);
    ms.up.save_a = at<void>(saved, sl.A);
    ms.up.save_b = at<void>(saved, sl.B);
    ms.up.save = (c.flags & MOK_FLAG_SAVE_FOR_BACKWARD) ? 1 : 0;
    ms.down = g;
    ms.down.A = at<void>(saved, sl.H);
    ms.down.B0 = W2;
    ms.down.out0 = at<void>(saved, sl.Y);
    ms.x = x;
    ms.pair_of_row = s_por;
    ms.k = k;
    ms.movers = c.mover_cus;
    ms.ctr = at<int32_t>(workspace, wl.queue) + 32;  // past the backward's 16 queue counters
    static_assert(32 + kRingCounters <= 64, "queue region");
    mark_empty_stage(c, s, MOK_STAGE_DISPATCH);
    MOK_HIP(launch_ring_reset(ms.ctr, s));
    {
      StageMark mark(c, s, MOK_STAGE_GEMM_UP);  // the whole pipeline
      for (int m = -1; m <= M; ++m) {
        ms.up0 = ms.up1 = ms.dn0 = ms.dn1 = ms.cp0 = ms.cp1 = 0;
        if (m >= 0 && m < M) {
          ms.up0 = m * R;
          ms.up1 = m * R + R;
          ms.up.a_row_shift = (int64_t)m * R - (int64_t)(m % S) * R;
        }
        if (m >= 1) {
          ms.dn0 = (m - 1) * R;
          ms.dn1 = m * R;
        }
        if (m + 1 < M) {
          ms.cp0 = (m + 1) * R;
          ms.cp1 = (m + 1) * R + R;
          ms.ring_dst = ring + (int64_t)((m + 1) % S) * R * d;
        }
        MOK_HIP(launch_minibatch_step(ms, s));
      }
    }
    mark_empty_stage(c, s, MOK_STAGE_GEMM_DOWN);
  } else {
    void* xp = at<void>(workspace, wl.xp);
    if (fused_pull(c)) {
      mark_empty_stage(c, s, MOK_STAGE_DISPATCH);
      g.A = x;
      g.gather_rows = s_por;
      g.k_top = k;
      g.gather_src_rows = T;
    } else {
      MOK_STAGE(MOK_STAGE_DISPATCH, launch_dispatch_gather(x, s_rop, T, k, d, bf16, xp, wl.xp_rows, status, s));
      g.A = xp;
    }
    g.B0 = W1;
    g.B1 = W3;
    g.out0 = at<void>(saved, sl.H);
    g.save_a = at<void>(saved, sl.A);
    g.save_b = at<void>(saved, sl.B);
    g.save = (c.flags & MOK_FLAG_SAVE_FOR_BACKWARD) ? 1 : 0;
    const bool stream = streaming_gemms(c, k);
    MOK_STAGE(MOK_STAGE_GEMM_UP, stream ? gemm_stream_bf16(KIND_UP, g, s) : run_gemm(c.precision, KIND_UP, g, s));
    GroupedGemmArgs g2 = g;
    g2.A = at<void>(saved, sl.H);
    g2.B0 = W2;
    g2.B1 = nullptr;
    g2.out0 = at<void>(saved, sl.Y);
    g2.save = 0;
    g2.gather_rows = nullptr;
    MOK_STAGE(MOK_STAGE_GEMM_DOWN,
              stream ? gemm_stream_bf16(KIND_DOWN, g2, s) : run_gemm(c.precision, KIND_DOWN, g2, s));
  }
  MOK_STAGE(MOK_STAGE_COMBINE, launch_combine(at<void>(saved, sl.Y), s_gate, s_rop, T, k, d, bf16, all_local(c), out,
                                              P_max, status, s));
  return MOK_OK;
}

// ------------------------------------------------------------ no-allocation forward
// mok_moe_forward_noalloc keeps its scratch (the status words and the counting
// sort's chunk tables) in this array instead of a caller's workspace.  One copy
// per GPU, held until the process ends; every call on a GPU shares it.
constexpr size_t kScratchBytes = size_t(4) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The array's device address on each GPU, taken once per device with that
// device current (the name itself is only a host-side stand-in).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

mok_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOK_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOK_ERR_HIP;
    size_t bytes = 0;  // the symbol found is the whole array
    if (hipGetSymbolSize(&bytes, HIP_SYMBOL(scratch)) != hipSuccess || bytes != kScratchBytes) return MOK_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOK_OK;
}

// Scratch of a bf16 whole-layer forward whose dispatch is fused into UP's
// loads: the status words and the two chunk tables of the counting sort.
WorkspaceLayout compact_forward_layout(const mok_moe_config& c, int32_t k) {
  WorkspaceLayout w{};
  const int64_t nchunks = ((int64_t)c.T * k + kSortChunk - 1) / kSortChunk;
  w.nchunks = (int)nchunks;
  size_t o = 0;
  w.status = o;        o = align256(o + 256);
  w.chunk_counts = o;  o = align256(o + (size_t)nchunks * c.E * 4);
  w.chunk_base = o;    o = align256(o + (size_t)nchunks * c.E * 4);
  w.tile_prefix = w.xp = w.xp_scale = w.hq = w.hq_scale = w.dy = w.dab = w.dxp = w.queue = w.wq = w.wq_scale = o;
  w.xp_rows = 0;
  w.total = o;
  return w;
}

}  // namespace

extern "C" {

const char* mok_status_string(mok_status s) {
  switch (s) {
    case MOK_OK: return "MOK_OK";
    case MOK_ERR_INVALID_ARG: return "MOK_ERR_INVALID_ARG: invalid argument (null pointer, shape or alignment)";
    case MOK_ERR_UNSUPPORTED: return "MOK_ERR_UNSUPPORTED: request not implemented by this library";
    case MOK_ERR_WORKSPACE: return "MOK_ERR_WORKSPACE: ring buffer smaller than two minibatch slots";
    case MOK_ERR_HIP: return "MOK_ERR_HIP: a HIP runtime call failed";
    case MOK_ERR_DEVICE: return "MOK_ERR_DEVICE: a device-side check failed";
  }
  return "unknown mok_status";
}

int32_t mok_version(void) { return 100; }

mok_status mok_moe_workspace_query(const mok_moe_config* cfg, int32_t k, size_t* workspace_bytes,
                                   size_t* saved_bytes) {
  mok_status st = validate_config(cfg, k);
  if (st != MOK_OK) return st;
  if (!workspace_bytes || !saved_bytes) return MOK_ERR_INVALID_ARG;
  WorkspaceLayout w;
  workspace_layout(*cfg, k, &w);
  mok_saved_layout s;
  size_t tp, eo;
  saved_layout(*cfg, k, &s, &tp, &eo);
  *workspace_bytes = w.total;
  *saved_bytes = s.total;
  return MOK_OK;
}

mok_status mok_moe_workspace_layout(const mok_moe_config* cfg, int32_t k, mok_workspace_layout* out) {
  mok_status st = validate_config(cfg, k);
  if (st != MOK_OK) return st;
  if (!out) return MOK_ERR_INVALID_ARG;
  WorkspaceLayout w;
  workspace_layout(*cfg, k, &w);
  out->status = w.status;
  out->xp = w.xp;
  out->xp_scale = w.xp_scale;
  out->xp_rows = w.xp_rows;
  out->hq = w.hq;
  out->hq_scale = w.hq_scale;
  out->dy = w.dy;
  out->dab = w.dab;
  out->dxp = w.dxp;
  out->wq = w.wq;
  out->wq_scale = w.wq_scale;
  out->k_pad = w.k_pad;
  out->total = w.total;
  return MOK_OK;
}

mok_status mok_moe_saved_layout(const mok_moe_config* cfg, int32_t k, mok_saved_layout* out) {
  mok_status st = validate_config(cfg, k);
  if (st != MOK_OK) return st;
  if (!out) return MOK_ERR_INVALID_ARG;
  size_t tp, eo;
  saved_layout(*cfg, k, out, &tp, &eo);
  return MOK_OK;
}

mok_status mok_moe_forward(const void* x, const float* router_logits, const void* W1, const void* W3,
                           const void* W2, int32_t k, const mok_moe_config* cfg, const uint8_t* w_scales,
                           void* out, int32_t* topk_idx, float* topk_gate, int32_t* expert_counts,
                           int32_t* expert_offsets, void* saved, void* workspace, void* stream) {
  mok_status st = validate_config(cfg, k);
  if (st != MOK_OK) return st;
  const mok_moe_config& c = *cfg;
  const void* always[] = {W1, W3, W2, expert_counts, expert_offsets, saved, workspace};
  const void* per_token[] = {x, router_logits, out, topk_idx, topk_gate};
  for (const void* p : always)
    if (!p || !aligned16(p)) return MOK_ERR_INVALID_ARG;
  for (const void* p : per_token)
    if ((c.T > 0 && !p) || !aligned16(p)) return MOK_ERR_INVALID_ARG;
  const bool mx = c.precision == MOK_PREC_MXFP8 || c.precision == MOK_PREC_MXFP4;
  if (mx && !w_scales) return MOK_ERR_INVALID_ARG;
  if (!mx && w_scales) return MOK_ERR_INVALID_ARG;

  WorkspaceLayout wl;
  workspace_layout(c, k, &wl);
  return forward_checked(x, router_logits, W1, W3, W2, k, c, w_scales, out, topk_idx, topk_gate, expert_counts,
                         expert_offsets, saved, workspace, wl, stream);
}

mok_status mok_moe_forward_noalloc(const void* x, const float* router_logits, const void* W1, const void* W3,
                                   const void* W2, int32_t k, const mok_moe_config* cfg, void* out,
                                   int32_t* topk_idx, float* topk_gate, int32_t* expert_counts,
                                   int32_t* expert_offsets, void* saved, void* stream) {
  mok_status st = validate_config(cfg, k);
  if (st != MOK_OK) return st;
  const mok_moe_config& c = *cfg;
  // the bf16 whole layer with the dispatch fused into UP: no row buffer
  if (c.precision != MOK_PREC_BF16 || c.minibatch_rows != 0 || !fused_pull(c)) return MOK_ERR_UNSUPPORTED;
  const void* always[] = {W1, W3, W2, expert_counts, expert_offsets, saved};
  const void* per_token[] = {x, router_logits, out, topk_idx, topk_gate};
  for (const void* p : always)
    if (!p || !aligned16(p)) return MOK_ERR_INVALID_ARG;
  for (const void* p : per_token)
    if ((c.T > 0 && !p) || !aligned16(p)) return MOK_ERR_INVALID_ARG;
  const WorkspaceLayout wl = compact_forward_layout(c, k);
  if (wl.total > kScratchBytes) return MOK_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != MOK_OK) return st;
  return forward_checked(x, router_logits, W1, W3, W2, k, c, nullptr, out, topk_idx, topk_gate, expert_counts,
                         expert_offsets, saved, ws, wl, stream);
}

mok_status mok_moe_backward(const void* dout, const void* x, const float* router_logits, const void* W1,
                            const void* W3, const void* W2, int32_t k, const mok_moe_config* cfg,
                            const void* saved, void* dx, float* dW1, float* dW3, float* dW2, float* dgate,
                            float* drouter_logits, void* workspace, void* stream) {
  mok_status st = validate_config(cfg, k);
  if (st != MOK_OK) return st;
  const mok_moe_config& c = *cfg;
  const void* always[] = {W1, W3, W2, saved, dW1, dW3, dW2, workspace};
  const void* per_token[] = {dout, x, router_logits, dx, dgate, drouter_logits};
  for (const void* p : always)
    if (!p || !aligned16(p)) return MOK_ERR_INVALID_ARG;
  for (const void* p : per_token)
    if ((c.T > 0 && !p) || !aligned16(p)) return MOK_ERR_INVALID_ARG;
  if (c.precision == MOK_PREC_MXFP8 || c.precision == MOK_PREC_MXFP4) return MOK_ERR_UNSUPPORTED;
  if (!(c.flags & MOK_FLAG_SAVE_FOR_BACKWARD)) return MOK_ERR_INVALID_ARG;

  hipStream_t s = (hipStream_t)stream;
  const int T = c.T, E = c.E, d = c.d, F = c.ffn, eb = c.expert_begin, E_loc = c.expert_end - c.expert_begin;
  const int bf16 = c.precision != MOK_PREC_F32;
  mok_saved_layout sl;
  size_t tp_off, eo_off;
  saved_layout(c, k, &sl, &tp_off, &eo_off);
  WorkspaceLayout wl;
  workspace_layout(c, k, &wl);
  const int32_t* s_idx = at<int32_t>(saved, sl.topk_idx);
  const float* s_gate = at<float>(saved, sl.topk_gate);
  const float* s_lse = at<float>(saved, sl.lse);
  const int32_t* s_off = at<int32_t>(saved, sl.offsets);
  const int32_t* s_tp = at<int32_t>(saved, tp_off);
  const int32_t* s_order = at<int32_t>(saved, eo_off);
  const int32_t* s_rop = at<int32_t>(saved, sl.row_of_pair);
  int32_t* queue = at<int32_t>(workspace, wl.queue);
  void* dy = at<void>(workspace, wl.dy);
  void* dab = at<void>(workspace, wl.dab);
  void* dxp = at<void>(workspace, wl.dxp);
  void* xp = at<void>(workspace, wl.xp);
  int32_t* status = at<int32_t>(workspace, wl.status);
  const int64_t P_max = (int64_t)T * k;
  MOK_HIP(launch_status_reset(status, s));

  // reverse-combine with the router backward
  MOK_STAGE(MOK_STAGE_BWD_GATE, launch_backward_gate(dout, at<void>(saved, sl.Y), s_gate, s_idx, s_rop, router_logits, s_lse, T, k, E, d,
                               gating_of(c), bf16, dgate, drouter_logits, dy, queue, 16, nullptr, nullptr, 0,
                               P_max, status, s));
  GroupedGemmArgs g{};
  g.offsets = s_off;
  g.tile_prefix = s_tp;
  g.expert_order = s_order;
  g.eb = eb;
  g.E_loc = E_loc;
  g.d = d;
  g.F = F;
  g.P_max = (int64_t)T * k;
  // dH = dY W2 -> dA, dB
  g.A = dy;
  g.B0 = W2;
  g.save_a = const_cast<void*>(at<void>(saved, sl.A));
  g.save_b = const_cast<void*>(at<void>(saved, sl.B));
  g.out0 = dab;
  MOK_STAGE(MOK_STAGE_GEMM_DH, run_gemm(c.precision, KIND_DH, g, s));
  // dX_perm = dA W1 + dB W3, then the reverse-dispatch reduction
  GroupedGemmArgs gx = g;
  gx.A = dab;
  gx.B0 = W1;
  gx.B1 = W3;
  gx.out0 = dxp;
  MOK_STAGE(MOK_STAGE_GEMM_DX, run_gemm(c.precision, KIND_DX, gx, s));
  MOK_STAGE(MOK_STAGE_REDUCE_DX, launch_combine(dxp, nullptr, s_rop, T, k, d, bf16, all_local(c), dx, P_max, status, s));
  // weight gradients
  GroupedGemmArgs gw = g;
  gw.A = dy;
  gw.B0 = at<void>(saved, sl.H);
  gw.out0 = dW2;
  gw.queue = queue;
  MOK_STAGE(MOK_STAGE_GEMM_DW2, run_gemm(c.precision, KIND_DW2, gw, s));
  GroupedGemmArgs g13 = g;
  g13.A = dab;
  if (c.minibatch_rows > 0) {
    // ring mode holds no expert-sorted copy of X: pull the token rows inside
    // the loads of the transposed operand
    mark_empty_stage(c, s, MOK_STAGE_REGATHER);
    g13.B0 = x;
    g13.gather_rows = at<int32_t>(saved, sl.pair_of_row);
    g13.k_top = k;
    g13.gather_src_rows = T;
  } else {
    // X rows again, expert-sorted (the transposed operand of dW1/dW3 wants
    // them contiguous: a gather inside its loads chains two loads)
    MOK_STAGE(MOK_STAGE_REGATHER, launch_dispatch_gather(x, s_rop, T, k, d, bf16, xp, wl.xp_rows, status, s));
    g13.B0 = xp;
  }
  g13.out0 = dW1;
  g13.out1 = dW3;
  g13.queue = queue + 8;
  MOK_STAGE(MOK_STAGE_GEMM_DW13, run_gemm(c.precision, KIND_DW13, g13, s));
  return MOK_OK;
}

mok_status mok_quantize_mxfp8(const void* src_bf16, int64_t rows, int64_t K, uint8_t* dst_e4m3, uint8_t* dst_e8m0,
                              void* stream) {
  if (rows < 0 || K <= 0 || K % 64) return MOK_ERR_INVALID_ARG;
  if (rows * (K / 32) >= (int64_t(1) << 32)) return MOK_ERR_INVALID_ARG;  // scale planes addressed in 32 bits
  if (rows == 0) return MOK_OK;
  if (!src_bf16 || !dst_e4m3 || !dst_e8m0 || !aligned16(src_bf16) || !aligned16(dst_e4m3)) return MOK_ERR_INVALID_ARG;
  MOK_HIP(launch_quantize_mxfp8(src_bf16, rows, K, dst_e4m3, dst_e8m0, (hipStream_t)stream));
  return MOK_OK;
}

mok_status mok_quantize_mxfp4(const void* src_bf16, int64_t rows, int64_t K, uint8_t* dst_e2m1, uint8_t* dst_e8m0,
                              void* stream) {
  if (rows < 0 || K <= 0 || K % 64) return MOK_ERR_INVALID_ARG;
  if (rows * (K / 32) >= (int64_t(1) << 32)) return MOK_ERR_INVALID_ARG;  // scale planes addressed in 32 bits
  if (rows == 0) return MOK_OK;
  if (!src_bf16 || !dst_e2m1 || !dst_e8m0 || !aligned16(src_bf16) || !aligned16(dst_e2m1)) return MOK_ERR_INVALID_ARG;
  MOK_HIP(launch_quantize_mxfp4(src_bf16, rows, K, dst_e2m1, dst_e8m0, (hipStream_t)stream));
  return MOK_OK;
}

mok_status mok_quantize_mxfp8_backward_weights(const void* W1, const void* W3, const void* W2, int32_t E_loc,
                                               int32_t d, int32_t F, uint8_t* wt_e4m3, uint8_t* wt_e8m0,
                                               void* stream) {
  if (E_loc < 1 || d <= 0 || F <= 0 || d % 128 || F % 128) return MOK_ERR_INVALID_ARG;
  const int64_t n = (int64_t)E_loc * F * d;  // elements of one weight tensor
  if (n / 32 * 2 >= (int64_t(1) << 32)) return MOK_ERR_INVALID_ARG;
  const void* ptrs[] = {W1, W3, W2, wt_e4m3, wt_e8m0};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MOK_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  // W2^T: [E_loc, F, d] along d; scale rows E_loc * F
  MOK_HIP(launch_quantize_mxfp8_t(W2, E_loc, d, F, wt_e4m3, (int64_t)F * d, d, 0, wt_e8m0, (int64_t)E_loc * F, s));
  // [W1^T | W3^T]: [E_loc, d, 2F] along 2F; scale rows E_loc * d
  uint8_t* q13 = wt_e4m3 + n;
  uint8_t* s13 = wt_e8m0 + n / 32;
  MOK_HIP(launch_quantize_mxfp8_t(W1, E_loc, F, d, q13, (int64_t)d * 2 * F, 2 * F, 0, s13, (int64_t)E_loc * d, s));
  MOK_HIP(launch_quantize_mxfp8_t(W3, E_loc, F, d, q13, (int64_t)d * 2 * F, 2 * F, F, s13, (int64_t)E_loc * d, s));
  return MOK_OK;
}

mok_status mok_moe_backward_mxfp8(const void* dout, const void* x, const float* router_logits, int32_t k,
                                  const mok_moe_config* cfg, const uint8_t* wt_e4m3,
                                  const uint8_t* wt_e8m0, const void* saved, void* dx, float* dW1,
                                  float* dW3, float* dW2, float* dgate, float* drouter_logits,
                                  void* workspace, void* stream) {
  mok_status st = validate_config(cfg, k);
  if (st != MOK_OK) return st;
  const mok_moe_config& c = *cfg;
  if (c.precision != MOK_PREC_MXFP8 || !(c.flags & MOK_FLAG_SAVE_FOR_BACKWARD)) return MOK_ERR_INVALID_ARG;
  const void* always[] = {wt_e4m3, wt_e8m0, saved, dW1, dW3, dW2, workspace};
  const void* per_token[] = {dout, x, router_logits, dx, dgate, drouter_logits};
  for (const void* p : always)
    if (!p || !aligned16(p)) return MOK_ERR_INVALID_ARG;
  for (const void* p : per_token)
    if ((c.T > 0 && !p) || !aligned16(p)) return MOK_ERR_INVALID_ARG;

  hipStream_t s = (hipStream_t)stream;
  const int T = c.T, E = c.E, d = c.d, F = c.ffn, eb = c.expert_begin, E_loc = c.expert_end - c.expert_begin;
  mok_saved_layout sl;
  size_t tp_off, eo_off;
  saved_layout(c, k, &sl, &tp_off, &eo_off);
  WorkspaceLayout wl;
  workspace_layout(c, k, &wl);
  const int32_t* s_idx = at<int32_t>(saved, sl.topk_idx);
  const float* s_gate = at<float>(saved, sl.topk_gate);
  const float* s_lse = at<float>(saved, sl.lse);
  const int32_t* s_rop = at<int32_t>(saved, sl.row_of_pair);
  int32_t* queue = at<int32_t>(workspace, wl.queue);
  void* dy = at<void>(workspace, wl.dy);
  void* dab = at<void>(workspace, wl.dab);
  void* dxp = at<void>(workspace, wl.dxp);
  uint8_t* dyq = at<uint8_t>(workspace, wl.xp);          // [P_max, d] codes
  uint8_t* dys = at<uint8_t>(workspace, wl.xp_scale);    // [d/64, P_max, 2]
  uint8_t* dabq = at<uint8_t>(workspace, wl.hq);         // [P_max, 2F] codes
  uint8_t* dabs = at<uint8_t>(workspace, wl.hq_scale);   // [2F/64, P_max, 2]
  const int64_t n = (int64_t)E_loc * F * d;
  int32_t* status = at<int32_t>(workspace, wl.status);
  const int64_t P_max = (int64_t)T * k;
  MOK_HIP(launch_status_reset(status, s));

  // reverse-combine with the router backward; dY also as MXFP8 along d
  MOK_STAGE(MOK_STAGE_BWD_GATE, launch_backward_gate(dout, at<void>(saved, sl.Y), s_gate, s_idx, s_rop, router_logits,
                                                      s_lse, T, k, E, d, gating_of(c), 1, dgate, drouter_logits,
                                                      (c.flags & MOK_FLAG_MXFP8_WGRAD) ? nullptr : dy,
                                                      queue, 16, dyq, dys, wl.xp_rows, P_max, status, s));
  GroupedGemmArgs g{};
  g.offsets = at<int32_t>(saved, sl.offsets);
  g.tile_prefix = at<int32_t>(saved, tp_off);
  g.expert_order = at<int32_t>(saved, eo_off);
  g.eb = eb;
  g.E_loc = E_loc;
  g.d = d;
  g.F = F;
  g.P_max = (int64_t)T * k;
  // dH = Q(dY) Q(W2^T)^T -> dA, dB (bf16) and [dA | dB] quantised along F
  GroupedGemmArgs gh = g;
  gh.A = dyq;
  gh.a_scale = dys;
  gh.B0 = wt_e4m3;
  gh.b_scale0 = wt_e8m0;
  gh.save_a = const_cast<void*>(at<void>(saved, sl.A));
  gh.save_b = const_cast<void*>(at<void>(saved, sl.B));
  gh.out0 = dab;
  gh.out1 = dabq;
  gh.out_scale = dabs;
  MOK_STAGE(MOK_STAGE_GEMM_DH, gemm_mxfp8(KIND_DH, gh, s));
  // dX_perm = Q([dA | dB]) Q([W1^T | W3^T])^T, then the reverse-dispatch sum
  GroupedGemmArgs gx = g;
  gx.A = dabq;
  gx.a_scale = dabs;
  gx.B0 = wt_e4m3 + n;
  gx.b_scale0 = wt_e8m0 + n / 32;
  gx.out0 = dxp;
  MOK_STAGE(MOK_STAGE_GEMM_DX, gemm_mxfp8(KIND_DX, gx, s));
  MOK_STAGE(MOK_STAGE_REDUCE_DX, launch_combine(dxp, nullptr, s_rop, T, k, d, 1, all_local(c), dx, P_max, status, s));
  if (c.flags & MOK_FLAG_MXFP8_WGRAD) {
    // weight gradients in MXFP8: dY, H, [dA | dB] and the x rows quantised
    // along each expert's rows (transposed codes), then the scaled-MFMA
    // products into the fp32 dW
    const int64_t kp = wl.k_pad;
    uint8_t* q = at<uint8_t>(workspace, wl.wq);
    uint8_t* qs = at<uint8_t>(workspace, wl.wq_scale);
    uint8_t *dyT = q, *hT = dyT + d * kp, *abT = hT + F * kp, *xT = abT + 2 * F * kp;
    uint8_t *dyS = qs, *hS = dyS + d * kp / 32, *abS = hS + F * kp / 32, *xS = abS + 2 * F * kp / 32;
    const int32_t* offs = at<int32_t>(saved, sl.offsets);
    const int32_t* tp128 = at<int32_t>(saved, tp_off) + 1 * (E_loc + 1);
    const int32_t* s_por = at<int32_t>(saved, sl.pair_of_row);
    const void* Hs = at<void>(saved, sl.H);
    // dY is formed again from dout and the gates (the reverse-combine's
    // product and rounding), which reads T rows of dout instead of P of dY
    const QrJob jobs[4] = {
        {(const uint16_t*)dout, d, s_por, s_gate, d, dyT, dyS},
        {(const uint16_t*)Hs, F, nullptr, nullptr, F, hT, hS},
        {(const uint16_t*)dab, 2 * F, nullptr, nullptr, 2 * F, abT, abS},
        {(const uint16_t*)x, d, s_por, nullptr, d, xT, xS}};
    MOK_STAGE(MOK_STAGE_REGATHER, launch_quantize_rows_t(jobs, 4, k, offs, eb, E_loc, tp128, P_max, kp, s));
    GroupedGemmArgs w2 = g;
    w2.k_pad = kp;
    w2.A = dyT;
    w2.a_scale = dyS;
    w2.B0 = hT;
    w2.b_scale0 = hS;
    w2.out0 = dW2;
    MOK_STAGE(MOK_STAGE_GEMM_DW2, gemm_mxfp8(KIND_DW2, w2, s));
    GroupedGemmArgs w13 = g;
    w13.k_pad = kp;
    w13.A = abT;
    w13.a_scale = abS;
    w13.B0 = xT;
    w13.b_scale0 = xS;
    w13.out0 = dW1;
    w13.out1 = dW3;
    MOK_STAGE(MOK_STAGE_GEMM_DW13, gemm_mxfp8(KIND_DW13, w13, s));
    return MOK_OK;
  }
  // weight gradients: bf16 products of the unquantised operands
  GroupedGemmArgs gw = g;
  gw.A = dy;
  gw.B0 = at<void>(saved, sl.H);
  gw.out0 = dW2;
  gw.queue = queue;
  MOK_STAGE(MOK_STAGE_GEMM_DW2, gemm_bf16(KIND_DW2, gw, s));
  // x rows again, expert-sorted, into dX_perm's buffer (read by the reduction
  // above, earlier on the stream)
  MOK_STAGE(MOK_STAGE_REGATHER, launch_dispatch_gather(x, s_rop, T, k, d, 1, dxp, P_max, status, s));
  GroupedGemmArgs g13 = g;
  g13.A = dab;
  g13.B0 = dxp;
  g13.out0 = dW1;
  g13.out1 = dW3;
  g13.queue = queue + 8;
  MOK_STAGE(MOK_STAGE_GEMM_DW13, gemm_bf16(KIND_DW13, g13, s));
  return MOK_OK;
}

}  // extern "C"

namespace {
// Token arrays (x, logits, dlogits, dx) may be NULL when T = 0.
mok_status validate_router(const void* x, const void* Wr, int32_t T, int32_t d, int32_t E) {
  if (T < 0 || T > (1 << 24) || d <= 0 || d % 64 || d > 65536 || E < 1 || E > 1024) return MOK_ERR_INVALID_ARG;
  if ((T > 0 && !x) || !Wr || !aligned16(x) || !aligned16(Wr)) return MOK_ERR_INVALID_ARG;
  return MOK_OK;
}
}  // namespace

extern "C" {

mok_status mok_router_logits(const void* x, const void* Wr, int32_t T, int32_t d, int32_t E, float* logits,
                             void* stream) {
  const mok_status st = validate_router(x, Wr, T, d, E);
  if (st != MOK_OK) return st;
  if (T == 0) return MOK_OK;
  if (!logits) return MOK_ERR_INVALID_ARG;
  MOK_HIP(launch_router_logits(x, Wr, T, d, E, logits, (hipStream_t)stream));
  return MOK_OK;
}

mok_status mok_moe_forward_router(const void* x, const void* Wr, const void* W1, const void* W3, const void* W2,
                                  int32_t k, const mok_moe_config* cfg, const uint8_t* w_scales, float* router_logits,
                                  void* out, int32_t* topk_idx, float* topk_gate, int32_t* expert_counts,
                                  int32_t* expert_offsets, void* saved, void* workspace, void* stream) {
  mok_status st = validate_config(cfg, k);
  if (st != MOK_OK) return st;
  const mok_moe_config& c = *cfg;
  if (c.precision == MOK_PREC_F32) return MOK_ERR_INVALID_ARG;  // the router GEMM takes bf16 x
  st = validate_router(x, Wr, c.T, c.d, c.E);
  if (st != MOK_OK) return st;
  const void* always[] = {W1, W3, W2, expert_counts, expert_offsets, saved, workspace};
  const void* per_token[] = {x, router_logits, out, topk_idx, topk_gate};
  for (const void* p : always)
    if (!p || !aligned16(p)) return MOK_ERR_INVALID_ARG;
  for (const void* p : per_token)
    if ((c.T > 0 && !p) || !aligned16(p)) return MOK_ERR_INVALID_ARG;
  const bool mx = c.precision == MOK_PREC_MXFP8 || c.precision == MOK_PREC_MXFP4;
  if (mx != (w_scales != nullptr)) return MOK_ERR_INVALID_ARG;
  WorkspaceLayout wl;
  workspace_layout(c, k, &wl);
  return forward_checked(x, router_logits, W1, W3, W2, k, c, w_scales, out, topk_idx, topk_gate, expert_counts,
                         expert_offsets, saved, workspace, wl, stream, Wr);
}

mok_status mok_router_logits_backward(const void* x, const void* Wr, const float* dlogits, int32_t T, int32_t d,
                                      int32_t E, float* dx, float* dWr, void* stream) {
  const mok_status st = validate_router(x, Wr, T, d, E);
  if (st != MOK_OK) return st;
  if ((T > 0 && (!dlogits || !dx)) || !dWr || !aligned16(dx) || !aligned16(dWr)) return MOK_ERR_INVALID_ARG;
  MOK_HIP(launch_router_logits_backward(x, Wr, dlogits, T, d, E, dx, dWr, (hipStream_t)stream));
  return MOK_OK;
}

}  // extern "C"
