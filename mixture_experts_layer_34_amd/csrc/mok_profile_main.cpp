// mok_profile: runs the MoE layer through the C ABI without PyTorch, for
// hardware-counter profiling (rocprofv3 --pmc) and standalone timing.
//
//   mok_profile [--T 8192] [--d 4096] [--E 128] [--k 8] [--F 1536] [--zipf 1.2]
//               [--steps 3] [--warmup 1] [--forward-only] [--copy-mib 0]
//               [--inputs DIR] [--mxfp8] [--mxfp8-wgrad]
//
// Inputs: with --inputs, the raw arrays that profile_inputs.py writes from the
// benchmark's own workload generator (x, logits, dout as bf16 / fp32 / bf16,
// W1, W3, W2 as bf16, row-major, native byte order), so that the counters
// are taken on exactly the benchmarked layer call.  Without it, synthetic
// values: x and weights hashed uniform values, router logits log(pi_e) +
// Gumbel noise with pi_r proportional to r^-zipf and expert 0 hottest (the
// same routing model; values and expert loads differ).  --mxfp8 runs the
// MXFP8 layer (weights quantised by mok_quantize_mxfp8 and
// mok_quantize_mxfp8_backward_weights before the timed steps); --mxfp8-wgrad
// also its weight gradients (MOK_FLAG_MXFP8_WGRAD).  --copy-mib
// runs one plain device copy kernel of that size first (HBM byte-counter
// calibration).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/mok.h"

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      exit(1);                                                                    \
    }                                                                             \
  } while (0)
#define MOKCHECK(x)                                                                \
  do {                                                                             \
    mok_status s_ = (x);                                                           \
    if (s_ != MOK_OK) {                                                            \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, mok_status_string(s_)); \
      exit(1);                                                                     \
    }                                                                              \
  } while (0)

__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16; x *= 0x7FEB352Du; x ^= x >> 15; x *= 0x846CA68Bu; x ^= x >> 16;
  return x;
}
__device__ __forceinline__ float unif(uint32_t seed, uint64_t i) {  // (0, 1)
  return ((hash32(seed ^ hash32((uint32_t)i ^ hash32((uint32_t)(i >> 32)))) >> 8) + 0.5f) * (1.0f / 16777216.0f);
}
// bf16 values uniform in [-a, a]
__global__ void fill_bf16(uint16_t* p, int64_t n, float a, uint32_t seed) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const float v = (2.0f * unif(seed, i) - 1.0f) * a;
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    p[i] = (uint16_t)(u >> 16);
  }
}
// logits[t, e] = log pi_e + Gumbel(0, 1)
__global__ void fill_logits(float* l, int T, int E, float s, float log_norm, uint32_t seed) {
  const int64_t n = (int64_t)T * E;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int e = (int)(i % E);
    l[i] = -s * logf((float)(e + 1)) - log_norm - logf(-logf(unif(seed, i)));
  }
}
__global__ void copy_kernel(const uint4* a, uint4* b, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) b[i] = a[i];
}

int main(int argc, char** argv) {
  int T = 8192, d = 4096, E = 128, k = 8, F = 1536, steps = 3, warmup = 1, copy_mib = 0;
  float zipf = 1.2f;
  bool backward = true, mxfp8 = false, mxfp8_wgrad = false;
  std::string inputs;
  for (int i = 1; i < argc; ++i) {
    std::string a = argv[i];
    auto next = [&]() { return (i + 1 < argc) ? argv[++i] : (fprintf(stderr, "missing value\n"), exit(2), ""); };
    if (a == "--T") T = atoi(next());
    else if (a == "--d") d = atoi(next());
    else if (a == "--E") E = atoi(next());
    else if (a == "--k") k = atoi(next());
    else if (a == "--F") F = atoi(next());
    else if (a == "--zipf") zipf = atof(next());
    else if (a == "--steps") steps = atoi(next());
    else if (a == "--warmup") warmup = atoi(next());
    else if (a == "--copy-mib") copy_mib = atoi(next());
    else if (a == "--forward-only") backward = false;
    else if (a == "--inputs") inputs = next();
    else if (a == "--mxfp8") mxfp8 = true;
    else if (a == "--mxfp8-wgrad") mxfp8 = mxfp8_wgrad = true;
    else { fprintf(stderr, "unknown argument %s\n", a.c_str()); return 2; }
  }
  if (copy_mib > 0) {
    const int64_t n = ((int64_t)copy_mib << 20) / 16;
    uint4 *a, *b;
    CHECK(hipMalloc(&a, n * 16));
    CHECK(hipMalloc(&b, n * 16));
    CHECK(hipMemset(a, 0, n * 16));
    hipLaunchKernelGGL(copy_kernel, dim3(4096), dim3(256), 0, 0, a, b, n);
    CHECK(hipDeviceSynchronize());
    CHECK(hipFree(a));
    CHECK(hipFree(b));
    printf("copy kernel: %d MiB read, %d MiB written\n", copy_mib, copy_mib);
  }
  mok_moe_config cfg;
  memset(&cfg, 0, sizeof(cfg));
  cfg.T = T; cfg.d = d; cfg.E = E; cfg.ffn = F; cfg.expert_begin = 0; cfg.expert_end = E;
  cfg.precision = mxfp8 ? MOK_PREC_MXFP8 : MOK_PREC_BF16;
  cfg.flags = backward ? MOK_FLAG_SAVE_FOR_BACKWARD : 0;
  if (mxfp8_wgrad && backward) cfg.flags |= MOK_FLAG_MXFP8_WGRAD;
  size_t ws_bytes, sv_bytes;
  MOKCHECK(mok_moe_workspace_query(&cfg, k, &ws_bytes, &sv_bytes));
  const int64_t xw = (int64_t)T * d, ww = (int64_t)E * F * d;
  uint16_t *x, *W1, *W3, *W2, *out, *dout, *dx;
  float *logits, *gate, *dW1, *dW3, *dW2, *dgate, *dlog;
  int32_t *idx, *counts, *offsets;
  void *saved, *ws;
  CHECK(hipMalloc(&x, xw * 2)); CHECK(hipMalloc(&out, xw * 2)); CHECK(hipMalloc(&dout, xw * 2)); CHECK(hipMalloc(&dx, xw * 2));
  CHECK(hipMalloc(&W1, ww * 2)); CHECK(hipMalloc(&W3, ww * 2)); CHECK(hipMalloc(&W2, ww * 2));
  CHECK(hipMalloc(&logits, (int64_t)T * E * 4)); CHECK(hipMalloc(&dlog, (int64_t)T * E * 4));
  CHECK(hipMalloc(&gate, (int64_t)T * k * 4)); CHECK(hipMalloc(&dgate, (int64_t)T * k * 4));
  CHECK(hipMalloc(&idx, (int64_t)T * k * 4)); CHECK(hipMalloc(&counts, E * 4)); CHECK(hipMalloc(&offsets, (E + 1) * 4));
  CHECK(hipMalloc(&dW1, ww * 4)); CHECK(hipMalloc(&dW3, ww * 4)); CHECK(hipMalloc(&dW2, ww * 4));
  CHECK(hipMalloc(&saved, sv_bytes)); CHECK(hipMalloc(&ws, ws_bytes));
  double norm = 0;
  for (int r = 1; r <= E; ++r) norm += std::pow((double)r, -(double)zipf);
  if (inputs.empty()) {
    hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, x, xw, 1.7f, 1u);
    hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, dout, xw, 1.7f, 2u);
    hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, W1, ww, 0.035f, 3u);
    hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, W3, ww, 0.035f, 4u);
    hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, W2, ww, 0.035f, 5u);
    hipLaunchKernelGGL(fill_logits, dim3(1024), dim3(256), 0, 0, logits, T, E, zipf, (float)std::log(norm), 6u);
  } else {
    // the raw arrays of the benchmark's workload, each checked for its exact size
    auto load = [&](const char* name, void* dst, int64_t bytes) {
      const std::string path = inputs + "/" + name;
      FILE* f = fopen(path.c_str(), "rb");
      if (!f) { fprintf(stderr, "cannot open %s\n", path.c_str()); exit(2); }
      std::vector<char> buf(bytes);
      const size_t got = fread(buf.data(), 1, bytes, f);
      const bool extra = fgetc(f) != EOF;
      fclose(f);
      if ((int64_t)got != bytes || extra) { fprintf(stderr, "%s: expected %lld bytes\n", path.c_str(), (long long)bytes); exit(2); }
      CHECK(hipMemcpy(dst, buf.data(), bytes, hipMemcpyHostToDevice));
    };
    load("x.bin", x, xw * 2);
    load("dout.bin", dout, xw * 2);
    load("logits.bin", logits, (int64_t)T * E * 4);
    load("W1.bin", W1, ww * 2);
    load("W3.bin", W3, ww * 2);
    load("W2.bin", W2, ww * 2);
  }
  CHECK(hipDeviceSynchronize());
  // MXFP8: forward weights along d (W1, W3) and F (W2), scales concatenated;
  // the backward's transposed copies
  uint8_t *q1 = nullptr, *q3 = nullptr, *q2 = nullptr, *wsc = nullptr, *wtq = nullptr, *wts = nullptr;
  if (mxfp8) {
    CHECK(hipMalloc(&q1, ww)); CHECK(hipMalloc(&q3, ww)); CHECK(hipMalloc(&q2, ww));
    CHECK(hipMalloc(&wsc, 3 * ww / 32));
    CHECK(hipMalloc(&wtq, 3 * ww)); CHECK(hipMalloc(&wts, 3 * ww / 32));
    MOKCHECK(mok_quantize_mxfp8(W1, (int64_t)E * F, d, q1, wsc, nullptr));
    MOKCHECK(mok_quantize_mxfp8(W3, (int64_t)E * F, d, q3, wsc + ww / 32, nullptr));
    MOKCHECK(mok_quantize_mxfp8(W2, (int64_t)E * d, F, q2, wsc + 2 * ww / 32, nullptr));
    MOKCHECK(mok_quantize_mxfp8_backward_weights(W1, W3, W2, E, d, F, wtq, wts, nullptr));
    CHECK(hipDeviceSynchronize());
  }
  auto step = [&]() {
    if (mxfp8) {
      MOKCHECK(mok_moe_forward(x, logits, q1, q3, q2, k, &cfg, wsc, out, idx, gate, counts, offsets, saved, ws,
                               nullptr));
      if (backward)
        MOKCHECK(mok_moe_backward_mxfp8(dout, x, logits, k, &cfg, wtq, wts, saved, dx, dW1, dW3, dW2, dgate, dlog,
                                        ws, nullptr));
      return;
    }
    MOKCHECK(mok_moe_forward(x, logits, W1, W3, W2, k, &cfg, nullptr, out, idx, gate, counts, offsets, saved, ws,
                             nullptr));
    if (backward)
      MOKCHECK(mok_moe_backward(dout, x, logits, W1, W3, W2, k, &cfg, saved, dx, dW1, dW3, dW2, dgate, dlog, ws,
                                nullptr));
  };
  for (int i = 0; i < warmup; ++i) step();
  // per-stage times of one extra step (events recorded by the library)
  std::vector<hipEvent_t> sev(2 * MOK_NUM_STAGES);
  for (auto& e : sev) CHECK(hipEventCreate(&e));
  cfg.stage_events = reinterpret_cast<void* const*>(sev.data());
  step();
  CHECK(hipDeviceSynchronize());
  cfg.stage_events = nullptr;
  static const char* names[MOK_NUM_STAGES] = {"router", "sort", "dispatch", "gemm_up", "gemm_down", "combine",
                                              "bwd_gate", "gemm_dh", "gemm_dx", "reduce_dx", "gemm_dw2",
                                              "regather", "gemm_dw13"};
  printf("stages (ms):");
  for (int st = 0; st < (backward ? (int)MOK_NUM_STAGES : 6); ++st) {
    float t = 0;
    CHECK(hipEventElapsedTime(&t, sev[2 * st], sev[2 * st + 1]));
    printf(" %s %.3f", names[st], t);
  }
  printf("\n");
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  CHECK(hipEventRecord(a, nullptr));
  for (int i = 0; i < steps; ++i) step();
  CHECK(hipEventRecord(b, nullptr));
  CHECK(hipEventSynchronize(b));
  float ms = 0;
  CHECK(hipEventElapsedTime(&ms, a, b));
  std::vector<int32_t> h_off(E + 1);
  CHECK(hipMemcpy(h_off.data(), offsets, (E + 1) * 4, hipMemcpyDeviceToHost));
  printf("T=%d d=%d E=%d k=%d F=%d zipf=%.2f %s %s%s: %.3f ms/step, P=%d\n", T, d, E, k, F, zipf,
         mxfp8 ? "mxfp8" : "bf16", backward ? "forward+backward" : "forward",
         inputs.empty() ? " (synthetic inputs)" : " (benchmark workload inputs)", ms / steps, h_off[E]);
  return 0;
}
