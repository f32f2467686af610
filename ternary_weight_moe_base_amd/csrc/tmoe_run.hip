// tmoe_run: a native driver of the library with no Python in the process.
//
// It draws a synthetic model in HBM through the C ABI (the counter-based
// weight generator, device ternarization and packing, tiled repacking), then
// runs one of three workloads on one stream and prints its timing:
//
//   tmoe_run layer  [--tokens T] [--layers L] [--steps N] [--warmup W] [--cfg C] [--host-experts 1]
//       tmoe_moe_forward over T tokens; step i runs layer i % L, so the packed
//       experts of consecutive steps are distinct HBM data. Weights are bit-
//       identical to those the Python package draws for the same cfg (same
//       Philox streams and key); activations come from the same generator on
//       a stream of their own (N(0,1) in the Irwin-Hall(12) approximation,
//       rounded to bf16). --host-experts 1 moves every layer's experts to
//       pinned host memory (tmoe_host_alloc) that the kernels read over PCIe.
//   tmoe_run lmhead [--tokens T] [--steps N] [--warmup W] [--vocab V] [--topk k]
//       tmoe_lm_head_topk over a [V][2048] bf16 table (fp32(0.02) * IH12,
//       rounded to bf16 on the device).
//   tmoe_run copy   [--mib M] [--steps N] [--host-experts 1]
//       a plain 16-byte-per-lane device copy of M MiB: the known-size kernel
//       that calibrates hardware byte counters; with --host-experts 1 the
//       source is pinned host memory (the host link's read rate).
//   tmoe_run issue
//       issue cost, in core-clock cycles per wavefront instruction and per
//       SIMD, of the instruction kinds the trit decode and the products are
//       made of (eight independent chains per wavefront, one and four
//       wavefronts per SIMD), of one product followed by V decode
//       instructions (whether the two overlap), and the core clock while
//       every SIMD of the chip issues packed fp16 FMAs: the figures that
//       turn a kernel's instruction counts into its issue-bound time.
//
// Model shape: hidden 2048, 256 experts, top-8, moe_intermediate 512 (the
// Maple-Preview configuration as the jj-blog architecture section and
// ai.thesatyajit.com, "The architecture around the quantization", give it).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <string>
#include <vector>

#include "tmoe.h"

namespace {

constexpr int64_t kH = 2048, kI = 512, kE = 256;
constexpr int kTopK = 8;
constexpr uint64_t kKey = 0x7E4A;  // generator key shared with the Python input module
constexpr int kMatGate = 0, kMatUp = 1, kMatDown = 2, kMatRouter = 3, kMatLmHead = 6, kMatActs = 7;

// Philox stream of one matrix: the numbering of the Python input module.
uint64_t stream_id(int cfg, int layer, int expert, int mat) {
  return 1 + ((((uint64_t)cfg * 64 + layer) * 1024 + expert) * 8 + mat);
}

#define CHECK_HIP(x)                                                                          \
  do {                                                                                     \
    hipError_t e_ = (x);                                                                   \
    if (e_ != hipSuccess) {                                                                \
      std::fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      std::exit(2);                                                                        \
    }                                                                                      \
  } while (0)
#define CHECK_TMOE(x)                                                                              \
  do {                                                                                          \
    int s_ = (x);                                                                               \
    if (s_ != TMOE_OK) {                                                                 \
      std::fprintf(stderr, "%s:%d: %s: %s (%s)\n", __FILE__, __LINE__, #x, tmoe_status_str(s_), \
                   tmoe_last_error());                                                          \
      std::exit(2);                                                                             \
    }                                                                                           \
  } while (0)

template <class T>
T *dalloc(size_t n) {
  void *p = nullptr;
  CHECK_HIP(hipMalloc(&p, n * sizeof(T) > 0 ? n * sizeof(T) : 1));
  return static_cast<T *>(p);
}

__global__ void copy16_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

// fp32 -> bf16, round to nearest even (finite inputs)
__global__ void to_bf16_kernel(const float *__restrict__ src, uint16_t *__restrict__ dst, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t u = __float_as_uint(src[i]);
    dst[i] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
  }
}

// ------------------------------------------------------------ issue costs
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kIssueKinds = 9;
const char *const kIssueNames[kIssueKinds] = {"v_pk_fma_f16", "v_pk_mad_u16", "v_pk_mul_lo_u16", "v_perm_b32",
                                              "v_add_u32",    "v_and_b32",    "v_lshlrev_b32",   "v_mov_b32",
                                              "v_fma_f32"};

// one instruction of kind KIND on x (ALU only)
template <int KIND>
__device__ __forceinline__ void issue_op(uint32_t &x, uint32_t k, uint32_t c) {
  if constexpr (KIND == 0) asm volatile("v_pk_fma_f16 %0, %0, %1, %2" : "+v"(x) : "s"(k), "v"(c));
  else if constexpr (KIND == 1) asm volatile("v_pk_mad_u16 %0, %0, %1, %2" : "+v"(x) : "s"(k), "v"(c));
  else if constexpr (KIND == 2) asm volatile("v_pk_mul_lo_u16 %0, %0, %1" : "+v"(x) : "s"(k));
  else if constexpr (KIND == 3) asm volatile("v_perm_b32 %0, %1, %0, %2" : "+v"(x) : "s"(k), "v"(c));
  else if constexpr (KIND == 4) asm volatile("v_add_u32 %0, %0, %1" : "+v"(x) : "v"(c));
  else if constexpr (KIND == 5) asm volatile("v_and_b32 %0, %0, %1" : "+v"(x) : "v"(c));
  else if constexpr (KIND == 6) asm volatile("v_lshlrev_b32 %0, 14, %0" : "+v"(x));
  else if constexpr (KIND == 7) asm volatile("v_mov_b32 %0, %1" : "+v"(x) : "v"(c));
  else asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x) : "s"(k), "v"(c));
}

// out[wave slot] = cycles of the timed loop, out[16384 + slot] = 100 MHz ticks
// of it; out[32768 + thread] keeps the chains live. The buffer holds
// 32768 + gridDim.x * blockDim.x words, gridDim.x <= 1024, blockDim.x <= 1024.
// MFMA: per unrolled step, MF products (four accumulators in turn) and V
// instructions of kind KIND.
template <int KIND, int V, int MF>
__global__ __launch_bounds__(1024) void issue_kernel(uint32_t *out, int iters, uint32_t k) {
  uint32_t a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = threadIdx.x + j;
  const uint32_t c = threadIdx.x ^ 0x1234u;
  bf16x8_t A, B;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    A[j] = (__bf16)(float)(threadIdx.x & 7);
    B[j] = (__bf16)(float)j;
  }
  f32x4_t acc[4] = {};
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int m = 0; m < MF; ++m) acc[m & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[m & 3], 0, 0, 0);
#pragma unroll
      for (int v = 0; v < V; ++v) issue_op<KIND>(a[v & 7], k, c);
    }
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  uint32_t r = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) r ^= a[j];
  const f32x4_t sacc = acc[0] + acc[1] + acc[2] + acc[3];
  out[32768 + blockIdx.x * blockDim.x + threadIdx.x] = r ^ __float_as_uint(sacc[0] + sacc[1] + sacc[2] + sacc[3]);
  if ((threadIdx.x & 63) == 0) {
    const int slot = blockIdx.x * 16 + (threadIdx.x >> 6);
    out[slot] = (uint32_t)(c1 - c0);
    out[16384 + slot] = (uint32_t)(r1 - r0);
  }
}

struct Args {
  std::string mode = "layer";
  int64_t tokens = 1;
  int layers = 24, steps = 240, warmup = 8, cfg = 2, topk = 16, host = 0;
  int64_t vocab = 151936, mib = 1024;
};

Args parse(int argc, char **argv) {
  Args a;
  int i = 1;
  if (argc > 1 && argv[1][0] != '-') a.mode = argv[i++];
  for (; i < argc; ++i) {
    const std::string k = argv[i];
    if (i + 1 >= argc) {
      std::fprintf(stderr, "missing value for %s\n", k.c_str());
      std::exit(1);
    }
    const long long v = std::atoll(argv[++i]);
    if (k == "--tokens") a.tokens = v;
    else if (k == "--layers") a.layers = (int)v;
    else if (k == "--steps") a.steps = (int)v;
    else if (k == "--warmup") a.warmup = (int)v;
    else if (k == "--cfg") a.cfg = (int)v;
    else if (k == "--vocab") a.vocab = v;
    else if (k == "--topk") a.topk = (int)v;
    else if (k == "--mib") a.mib = v;
    else if (k == "--host-experts") a.host = (int)v;
    else {
      std::fprintf(stderr, "unknown option %s\n", k.c_str());
      std::exit(1);
    }
  }
  if (a.tokens < 1 || a.layers < 1 || a.layers > 64 || a.steps < 1 || a.warmup < 0 || a.cfg < 0 || a.cfg > 63 ||
      a.mib < 1) {
    std::fprintf(stderr, "argument out of range\n");
    std::exit(1);
  }
  return a;
}

// One expert matrix [rows][cols]: raw weights -> ternary codes + row scales -> tiled packing.
void make_matrix(hipStream_t st, uint64_t sid, int64_t rows, int64_t cols, float *wbuf, uint8_t *pbuf, uint8_t *tiled,
                 float *scales) {
  CHECK_TMOE(tmoe_synth_ih12(st, kKey, 0, sid, 0, rows * cols, 1.0f, wbuf));
  const int64_t ldp = (cols + 4) / 5;
  CHECK_TMOE(tmoe_ternarize_pack(st, wbuf, rows, cols, pbuf, ldp, scales));
  CHECK_TMOE(tmoe_repack_tiled(st, pbuf, rows, cols, ldp, tiled));
}

void bf16_activations(hipStream_t st, uint64_t sid, int64_t n, float mult, uint16_t *out) {
  float *tmp = dalloc<float>(n);
  CHECK_TMOE(tmoe_synth_ih12(st, kKey, 0, sid, 0, n, mult, tmp));
  to_bf16_kernel<<<1024, 256, 0, st>>>(tmp, out, n);
  CHECK_HIP(hipGetLastError());
  CHECK_HIP(hipStreamSynchronize(st));
  CHECK_HIP(hipFree(tmp));
}

double time_loop(hipStream_t st, int warmup, int steps, const std::function<void(int)> &step) {
  for (int i = 0; i < warmup; ++i) step(i);
  CHECK_HIP(hipStreamSynchronize(st));
  hipEvent_t e0, e1;
  CHECK_HIP(hipEventCreate(&e0));
  CHECK_HIP(hipEventCreate(&e1));
  CHECK_HIP(hipEventRecord(e0, st));
  for (int i = 0; i < steps; ++i) step(warmup + i);
  CHECK_HIP(hipEventRecord(e1, st));
  CHECK_HIP(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK_HIP(hipEventElapsedTime(&ms, e0, e1));
  CHECK_HIP(hipEventDestroy(e0));
  CHECK_HIP(hipEventDestroy(e1));
  return 1e3 * ms / steps;
}

int run_layer(const Args &a, hipStream_t st) {
  const int64_t sgu = tmoe_tiled_bytes(kI, kH), sd = tmoe_tiled_bytes(kH, kI);
  float *wbuf = dalloc<float>(kH * kI);
  uint8_t *pbuf = dalloc<uint8_t>(kH * ((kH + 4) / 5));
  std::vector<tmoe_moe_weights> W(a.layers);
  for (int l = 0; l < a.layers; ++l) {
    uint8_t *gp = dalloc<uint8_t>(kE * sgu), *up = dalloc<uint8_t>(kE * sgu), *dp = dalloc<uint8_t>(kE * sd);
    float *gs = dalloc<float>(kE * kI), *us = dalloc<float>(kE * kI), *ds = dalloc<float>(kE * kH);
    float *rw = dalloc<float>(kE * kH);
    for (int e = 0; e < kE; ++e) {
      make_matrix(st, stream_id(a.cfg, l, e, kMatGate), kI, kH, wbuf, pbuf, gp + e * sgu, gs + e * kI);
      make_matrix(st, stream_id(a.cfg, l, e, kMatUp), kI, kH, wbuf, pbuf, up + e * sgu, us + e * kI);
      make_matrix(st, stream_id(a.cfg, l, e, kMatDown), kH, kI, wbuf, pbuf, dp + e * sd, ds + e * kH);
    }
    CHECK_TMOE(tmoe_synth_ih12(st, kKey, 0, stream_id(a.cfg, l, 1023, kMatRouter), 0, kE * kH, 0.02f, rw));
    W[l] = tmoe_moe_weights{kH, kI, kE, kTopK, 0, rw, nullptr, gp, up, dp, sgu, sd, gs, us, ds};
    if (a.host) {  // experts to pinned host memory: [gate | up | down | gate_s | up_s | down_s]
      const int64_t sz[6] = {kE * sgu, kE * sgu, kE * sd, 4 * kE * kI, 4 * kE * kI, 4 * kE * kH};
      void *src[6] = {gp, up, dp, gs, us, ds};
      int64_t total = 0;
      for (int64_t b : sz) total += b;
      void *h = nullptr, *d = nullptr;
      CHECK_TMOE(tmoe_host_alloc((size_t)total, &h, &d));
      CHECK_HIP(hipStreamSynchronize(st));
      int64_t off = 0;
      const void *dst[6];
      for (int i = 0; i < 6; ++i) {
        CHECK_HIP(hipMemcpy(static_cast<char *>(h) + off, src[i], sz[i], hipMemcpyDeviceToHost));
        CHECK_HIP(hipFree(src[i]));
        dst[i] = static_cast<char *>(d) + off;
        off += sz[i];
      }
      W[l].gate_p = static_cast<const uint8_t *>(dst[0]);
      W[l].up_p = static_cast<const uint8_t *>(dst[1]);
      W[l].down_p = static_cast<const uint8_t *>(dst[2]);
      W[l].gate_s = static_cast<const float *>(dst[3]);
      W[l].up_s = static_cast<const float *>(dst[4]);
      W[l].down_s = static_cast<const float *>(dst[5]);
    }
  }
  CHECK_HIP(hipStreamSynchronize(st));
  uint16_t *X = dalloc<uint16_t>(a.tokens * kH);
  bf16_activations(st, stream_id(a.cfg, 0, 1022, kMatActs), a.tokens * kH, 1.0f, X);
  float *Y = dalloc<float>(a.tokens * kH);
  size_t wsb = 0;
  CHECK_TMOE(tmoe_moe_workspace_bytes(a.tokens, &W[0], &wsb));
  void *ws = dalloc<uint8_t>(wsb);
  CHECK_HIP(hipMemset(ws, 0, wsb));  // once: the layer leaves its bound slots at zero
  const double us = time_loop(st, a.warmup, a.steps, [&](int i) {
    CHECK_TMOE(tmoe_moe_forward(st, &W[i % a.layers], X, a.tokens, Y, nullptr, ws, wsb));
  });
  std::printf("layer: tokens %lld, %d distinct layers, experts in %s, %d steps: %.2f us/step, %.0f tokens/s\n",
              (long long)a.tokens, a.layers, a.host ? "pinned host memory" : "HBM", a.steps, us, a.tokens * 1e6 / us);
  return 0;
}

int run_lmhead(const Args &a, hipStream_t st) {
  uint16_t *table = dalloc<uint16_t>(a.vocab * kH);
  bf16_activations(st, stream_id(a.cfg, 0, 0, kMatLmHead), a.vocab * kH, 0.02f, table);
  uint16_t *X = dalloc<uint16_t>(a.tokens * kH);
  bf16_activations(st, stream_id(a.cfg, 0, 1022, kMatActs), a.tokens * kH, 1.0f, X);
  const size_t wsb = tmoe_lm_head_workspace_bytes(a.tokens, a.vocab, a.topk);
  if (wsb == 0) {
    std::fprintf(stderr, "lm head: unsupported sizes (%s)\n", tmoe_last_error());
    return 1;
  }
  void *ws = dalloc<uint8_t>(wsb);
  int32_t *idx = dalloc<int32_t>(a.tokens * a.topk), *nfix = dalloc<int32_t>(1);
  float *val = dalloc<float>(a.tokens * a.topk);
  const double us = time_loop(st, a.warmup, a.steps, [&](int) {
    CHECK_TMOE(tmoe_lm_head_topk(st, X, a.tokens, kH, table, a.vocab, a.topk, idx, val, nullptr, nfix, ws, wsb));
  });
  std::printf("lmhead: tokens %lld, vocab %lld, top-%d, %d steps: %.2f us/step\n", (long long)a.tokens,
              (long long)a.vocab, a.topk, a.steps, us);
  return 0;
}

int run_copy(const Args &a, hipStream_t st) {
  const int64_t bytes = a.mib << 20, n = bytes / 16;
  uint4 *src = nullptr, *dst = dalloc<uint4>(n);
  if (a.host) {
    void *h = nullptr, *d = nullptr;
    CHECK_TMOE(tmoe_host_alloc((size_t)bytes, &h, &d));
    std::memset(h, 1, bytes);
    src = static_cast<uint4 *>(d);
  } else {
    src = dalloc<uint4>(n);
    CHECK_HIP(hipMemsetAsync(src, 1, bytes, st));
  }
  const double us = time_loop(st, 1, a.steps, [&](int) {
    copy16_kernel<<<4096, 256, 0, st>>>(src, dst, n);
    CHECK_HIP(hipGetLastError());
  });
  std::printf("copy: %lld bytes read (from %s) and written per launch, %d launches: %.2f us, %.1f GB/s read\n",
              (long long)bytes, a.host ? "pinned host memory" : "HBM", a.steps, us, 1e-3 * bytes / us);
  return 0;
}

// Cycles per instruction per SIMD, the largest over the wavefronts of one
// workgroup on one CU (64 threads: one wavefront per SIMD in use; 1024: four).
template <int KIND, int V, int MF>
double issue_cycles(uint32_t *d, std::vector<uint32_t> &h, int threads, int iters, double per_step) {
  issue_kernel<KIND, V, MF><<<1, threads>>>(d, iters, 0x35553555u);
  CHECK_HIP(hipGetLastError());
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(h.data(), d, 16 * sizeof(uint32_t), hipMemcpyDeviceToHost));
  uint32_t mx = 0;
  for (int w = 0; w < threads / 64; ++w) mx = h[w] > mx ? h[w] : mx;
  const double waves_per_simd = threads >= 256 ? threads / 256.0 : 1.0;
  return (double)mx / (iters * 4.0 * per_step) / waves_per_simd;
}

template <int KIND>
void issue_row(uint32_t *d, std::vector<uint32_t> &h) {
  const double c1 = issue_cycles<KIND, 8, 0>(d, h, 64, 2000, 8), c4 = issue_cycles<KIND, 8, 0>(d, h, 1024, 2000, 8);
  std::printf("  %-22s %8.2f %8.2f\n", kIssueNames[KIND], c1, c4);
}

int run_issue() {
  uint32_t *d = dalloc<uint32_t>(32768 + 1024 * 1024);
  std::vector<uint32_t> h(32768);
  std::printf("issue cost, cycles per wavefront instruction per SIMD (8 independent chains per wavefront)\n");
  std::printf("  %-22s %8s %8s\n", "instruction", "1 wave", "4 waves");
  issue_row<0>(d, h);
  issue_row<1>(d, h);
  issue_row<2>(d, h);
  issue_row<3>(d, h);
  issue_row<4>(d, h);
  issue_row<5>(d, h);
  issue_row<6>(d, h);
  issue_row<7>(d, h);
  issue_row<8>(d, h);
  std::printf("  %-22s %8.2f %8.2f\n", "v_mfma_f32_16x16x32_bf16", issue_cycles<0, 0, 4>(d, h, 64, 1000, 4),
              issue_cycles<0, 0, 4>(d, h, 1024, 1000, 4));
  std::printf("one product + V v_pk_fma_f16, cycles per step per SIMD (4 waves): additive if = mfma + V x fma\n");
  std::printf("  V = 4: %.2f   V = 8: %.2f   V = 12: %.2f   V = 24: %.2f\n", issue_cycles<0, 4, 1>(d, h, 1024, 1000, 1),
              issue_cycles<0, 8, 1>(d, h, 1024, 1000, 1), issue_cycles<0, 12, 1>(d, h, 1024, 1000, 1),
              issue_cycles<0, 24, 1>(d, h, 1024, 1000, 1));
  // the core clock under a chip-wide packed fp16 FMA load
  const int wgs = 1024;
  issue_kernel<0, 8, 0><<<wgs, 1024>>>(d, 4000, 0x35553555u);
  CHECK_HIP(hipGetLastError());
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(h.data(), d, 32768 * sizeof(uint32_t), hipMemcpyDeviceToHost));
  double ghz_sum = 0.0;
  int nw = 0;
  for (int i = 0; i < wgs * 16; ++i)
    if (h[16384 + i] > 0) {
      ghz_sum += 0.1 * h[i] / h[16384 + i];
      ++nw;
    }
  std::printf("core clock under a chip-wide v_pk_fma_f16 load: %.3f GHz (mean over %d wavefronts)\n",
              nw ? ghz_sum / nw : 0.0, nw);
  CHECK_HIP(hipFree(d));
  return 0;
}

}  // namespace

int main(int argc, char **argv) {
  const Args a = parse(argc, argv);
  hipStream_t st;
  CHECK_HIP(hipStreamCreateWithFlags(&st, hipStreamNonBlocking));
  int rc = 1;
  if (a.mode == "layer") rc = run_layer(a, st);
  else if (a.mode == "lmhead") rc = run_lmhead(a, st);
  else if (a.mode == "copy") rc = run_copy(a, st);
  else if (a.mode == "issue") rc = run_issue();
  else std::fprintf(stderr, "unknown mode %s (layer | lmhead | copy | issue)\n", a.mode.c_str());
  CHECK_HIP(hipStreamSynchronize(st));
  CHECK_HIP(hipStreamDestroy(st));
  std::fflush(stdout);
  return rc;
}
