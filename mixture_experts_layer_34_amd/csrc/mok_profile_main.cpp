// mok_profile: runs the MoE layer through the C ABI without PyTorch, for
// hardware-counter profiling (rocprofv3 --pmc) and standalone timing.
//
//   mok_profile [--T 8192] [--d 4096] [--E 128] [--k 8] [--F 1536] [--zipf 1.2]
//               [--steps 3] [--warmup 1] [--forward-only] [--copy-mib 0]
//
// Inputs are synthetic: x and weights hashed uniform values (N(0,1)-like and
// N(0, 0.02^2)-like spread), router logits log(pi_e) + Gumbel noise with
// pi_r proportional to r^-zipf and expert 0 hottest — the same routing model
// as the training workload of the Python benchmark (values differ; shapes and
// expert loads follow the same distribution).  --copy-mib runs one plain
// device copy kernel of that size first (HBM byte-counter calibration).
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
  bool backward = true;
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
  cfg.precision = MOK_PREC_BF16;
  cfg.flags = backward ? MOK_FLAG_SAVE_FOR_BACKWARD : 0;
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
  hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, x, xw, 1.7f, 1u);
  hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, dout, xw, 1.7f, 2u);
  hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, W1, ww, 0.035f, 3u);
  hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, W3, ww, 0.035f, 4u);
  hipLaunchKernelGGL(fill_bf16, dim3(4096), dim3(256), 0, 0, W2, ww, 0.035f, 5u);
  hipLaunchKernelGGL(fill_logits, dim3(1024), dim3(256), 0, 0, logits, T, E, zipf, (float)std::log(norm), 6u);
  CHECK(hipDeviceSynchronize());
  auto step = [&]() {
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
  printf("T=%d d=%d E=%d k=%d F=%d zipf=%.2f %s: %.3f ms/step, P=%d\n", T, d, E, k, F, zipf,
         backward ? "forward+backward" : "forward", ms / steps, h_off[E]);
  return 0;
}
