// Full-precision router with a certified top-k.
//
// The router of each layer stays in full precision and selects 8 of 256
// experts from its logits (ai.thesatyajit.com, "The claim, verified from the
// bytes"; codeinsider.com.br, "256 experts, 8 ativos"). The selection must be
// that of the exact logits. Every product bf16 x fp32 is exact in fp64, so the
// logits are accumulated in fp64 (full rate on CDNA4); a rigorous bound on the
// summation error certifies the ranking, and the rare token it cannot certify
// (in practice: exactly equal logits) is recomputed in double-double.
//
// Error bound (Higham, "Accuracy and Stability of Numerical Algorithms",
// recursive summation with FMA): |fl(l_e) - l_e| <= gamma_d * (A_e + |b_e|),
// A_e = sum_i |x_i w_ei|, gamma_d = d u / (1 - d u), u = 2^-53, d = chain length
// + butterfly depth + 1 (bias) + margin. With A = max_e (A_e + |b_e|) (also
// accumulated in fp64, and inflated by 1%) one bound B = gamma_d A serves the
// whole token: the top k+1 ranking is certified when each adjacent gap > 2B.
#include "route_util.h"

namespace tmoe {

static constexpr int kTokChunkBytes = 65536;  // LDS bytes of bf16 activations per workgroup
static constexpr int kVectorRouterMaxT = 64;  // up to 64 tokens the VALU kernel beats the fp64 matrix cores

size_t router_ws_bytes(int64_t T, int64_t E) {
  size_t o = 0;
  o = align_up(o + T * cdiv(E, 4) * 8, 256);  // bnd
  o = align_up(o + T * E * 8, 256);  // lg
  return o;
}

RouterWs router_ws_carve(void *ws, int64_t T, int64_t E) {
  char *b = (char *)ws;
  RouterWs r;
  size_t o = 0;
  r.bnd = (uint64_t *)(b + o);
  o = align_up(o + T * cdiv(E, 4) * 8, 256);
  r.lg = (double *)(b + o);
  return r;
}

// ------------------------------------------------------------ fp64 logits
// Each lane keeps 4*NC router weights (elements c*256 + 4*lane + 0..3) as fp64
// and runs one FMA chain of 4*NC exact products per logit, then a 6-level
// butterfly: depth 4*NC + 6, plus 1 for the bias. The same chain accumulates
// A = sum |x w| for the bound. Results for token n go to lgs[n*4 + wave] and
// abs_s[n*4 + wave] (LDS).
template <int NC>
__device__ inline void logits_rows(const uint16_t *xs, int nt, const float *Wr, const float *bias, int64_t e, int E,
                                   double *lgs, double *abs_s) {
  constexpr int H = NC * 256;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (e >= E) {
    if (lane < nt) {
      for (int n = lane; n < nt; n += 64) {
        lgs[n * 4 + wave] = 0.0;
        abs_s[n * 4 + wave] = 0.0;
      }
    }
    return;
  }
  double w[4 * NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float4 v = reinterpret_cast<const float4 *>(Wr + e * H)[c * 64 + lane];
    w[4 * c] = v.x;
    w[4 * c + 1] = v.y;
    w[4 * c + 2] = v.z;
    w[4 * c + 3] = v.w;
  }
  const double b = bias ? (double)bias[e] : 0.0;
  for (int n = 0; n < nt; ++n) {
    const uint2 *xr = reinterpret_cast<const uint2 *>(xs + (size_t)n * H);
    double acc = 0.0, aab = 0.0;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint2 xv = xr[c * 64 + lane];
      const double x0 = __uint_as_float(xv.x << 16), x1 = __uint_as_float(xv.x & 0xFFFF0000u);
      const double x2 = __uint_as_float(xv.y << 16), x3 = __uint_as_float(xv.y & 0xFFFF0000u);
      acc = fma(w[4 * c], x0, acc);
      acc = fma(w[4 * c + 1], x1, acc);
      acc = fma(w[4 * c + 2], x2, acc);
      acc = fma(w[4 * c + 3], x3, acc);
      aab = fma(fabs(w[4 * c]), fabs(x0), aab);
      aab = fma(fabs(w[4 * c + 1]), fabs(x1), aab);
      aab = fma(fabs(w[4 * c + 2]), fabs(x2), aab);
      aab = fma(fabs(w[4 * c + 3]), fabs(x3), aab);
    }
    acc = wave_sum_d(acc);
    aab = wave_sum_d(aab);
    if (lane == 0) {
      lgs[n * 4 + wave] = acc + b;
      abs_s[n * 4 + wave] = aab + fabs(b);
    }
  }
}

__device__ inline void stage_x(uint16_t *xs, const uint16_t *X, int64_t t0, int nt, int H) {
  const int vpr = H / 8;
  copy16<256>(
      nt * vpr, [&](int i) { return reinterpret_cast<const uint4 *>(X + t0 * H)[i]; },
      [&](int i) { return reinterpret_cast<uint4 *>(xs) + i; });
}

// Workgroup = 4 wavefronts = 4 experts; grid.y walks token chunks.
template <int NC>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t *X, int64_t T, const float *Wr,
                                                            const float *bias, int64_t E, int tchunk, double *lg,
                                                            uint64_t *bnd, int32_t *n_fixup) {
  extern __shared__ __align__(16) uint16_t xs[];
  __shared__ double lgs[4 * 128], abs_s[4 * 128];
  const int64_t e0 = (int64_t)blockIdx.x * 4;
  const int64_t t0 = (int64_t)blockIdx.y * tchunk;
  const int nt = (int)min<int64_t>(tchunk, T - t0);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0 && n_fixup) *n_fixup = 0;
  stage_x(xs, X, t0, nt, NC * 256);
  __syncthreads();
  logits_rows<NC>(xs, nt, Wr, bias, e0 + (threadIdx.x >> 6), (int)E, lgs, abs_s);
  __syncthreads();
  for (int i = threadIdx.x; i < nt * 4; i += 256) {
    const int n = i >> 2, q = i & 3;
    if (e0 + q < E) lg[(t0 + n) * E + e0 + q] = lgs[i];
  }
  for (int n = threadIdx.x; n < nt; n += 256) {
    const double a = fmax(fmax(abs_s[n * 4], abs_s[n * 4 + 1]), fmax(abs_s[n * 4 + 2], abs_s[n * 4 + 3]));
    bnd[(t0 + n) * gridDim.x + blockIdx.x] = dbits(a);  // this workgroup's bound slot of token t0 + n
  }
}

// ------------------------------------------------- fp64 matrix-core logits
// Batched logits: workgroup = 16 tokens x 16 experts, wavefront w accumulates
// the input range [w H/4, (w+1) H/4) on the fp64 matrix core (16x16x4: lane l
// supplies token / expert l mod 16 at input kb(l / 16) + step, each lane group
// owning a contiguous run of H/16 inputs). Every product bf16 x fp32 is exact
// in fp64; the four partial sums are added in fixed order (+ bias). The error
// bound uses Cauchy-Schwarz, sum_i |x_i w_ei| <= |x|_2 |w_e|_2, with the norms
// accumulated in fp64 alongside, and the depth of a sequential sum over H
// inputs (an upper bound for any order the matrix core adds in).
template <int NC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void router_mfma_kernel(const uint16_t *X, int64_t T, const float *Wr,
                                                          const float *bias, int E, double *lg, uint64_t *bnd,
                                                          int32_t *n_fixup) {
  constexpr int H = NC * 256;
  __shared__ double part[4][64][4];
  __shared__ double nx2[4][16], nw2[4][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.y * 16;
  const int e0 = blockIdx.x * 16;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0 && n_fixup) *n_fixup = 0;
  const bool tv = t0 + i < T, ev = e0 + i < E;  // rows past T / E read row 0 and are not stored
  constexpr int kl = H / 16;
  const int kb = wave * (H / 4) + g * kl;
  const uint16_t *xr = X + (tv ? t0 + i : 0) * (int64_t)H + kb;
  const float *wr = Wr + (int64_t)(ev ? e0 + i : 0) * H + kb;
  // four independent accumulation chains (steps j mod 4), added in fixed order at the end
  f64x4 acc4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc4[q] = f64x4{0.0, 0.0, 0.0, 0.0};
  // squared norms in fp32 (bf16 squares are exact; the fp32 sums are within
  // 1 + 2^-12 of the exact ones for H <= 4096, covered by the 1.01 margin)
  float sx = 0.f, sw = 0.f;
  // every load of the lane's run is issued before the first product
  constexpr int NCH = kl / 8;
  uint4 xv[NCH];
  float4 wv[2 * NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    xv[c] = *reinterpret_cast<const uint4 *>(xr + 8 * c);
    wv[2 * c] = *reinterpret_cast<const float4 *>(wr + 8 * c);
    wv[2 * c + 1] = *reinterpret_cast<const float4 *>(wr + 8 * c + 4);
  }
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const uint32_t xw[4] = {xv[c].x, xv[c].y, xv[c].z, xv[c].w};
    const float wf[8] = {wv[2 * c].x, wv[2 * c].y, wv[2 * c].z, wv[2 * c].w,
                         wv[2 * c + 1].x, wv[2 * c + 1].y, wv[2 * c + 1].z, wv[2 * c + 1].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // rows past T / E read row 0 (clamped pointers): their results are not stored
      const float xf = __uint_as_float((j & 1) ? (xw[j >> 1] & 0xFFFF0000u) : (xw[j >> 1] << 16));
      acc4[j & 3] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xf, (double)wf[j], acc4[j & 3], 0, 0, 0);
      sx = fmaf(xf, xf, sx);
      sw = fmaf(wf[j], wf[j], sw);
    }
  }
  const f64x4 acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
  // squared norms of token / expert i over this wavefront's inputs
  sx += __shfl_xor(sx, 16, 64);
  sx += __shfl_xor(sx, 32, 64);
  sw += __shfl_xor(sw, 16, 64);
  sw += __shfl_xor(sw, 32, 64);
  if (g == 0) {
    nx2[wave][i] = (double)sx;
    nw2[wave][i] = (double)sw;
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) part[wave][lane][v] = acc[v];
  __syncthreads();
  if (wave == 0) {
    // the fp64 16x16x4 result: lane l holds tokens t0 + l/16 + 4v, expert e0 + l%16
    const int e = e0 + i;
    const double b = (bias && e < E) ? (double)bias[e] : 0.0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t t = t0 + g + 4 * v;
      const double d = ((part[0][lane][v] + part[1][lane][v]) + part[2][lane][v]) + part[3][lane][v];
      if (t < T && e < E) lg[t * E + e] = d + b;
    }
  } else if (wave == 1 && lane < 16) {
    // per-token bound contribution: max over this workgroup's experts of |x_t| |w_e| + |b_e|
    const int64_t t = t0 + lane;
    if (t < T) {
      const double nx = sqrt(((nx2[0][lane] + nx2[1][lane]) + nx2[2][lane]) + nx2[3][lane]);
      double m = 0.0;
      for (int j = 0; j < 16 && e0 + j < E; ++j) {
        const double nw = sqrt(((nw2[0][j] + nw2[1][j]) + nw2[2][j]) + nw2[3][j]);
        m = fmax(m, nx * nw + (bias ? fabs((double)bias[e0 + j]) : 0.0));
      }
      bnd[t * gridDim.x + blockIdx.x] = dbits(m);  // this workgroup's bound slot of token t
    }
  }
}

// One wavefront per token: certified top-k from the fp64 logits, else the
// double-double recompute (counted in *n_fixup).
template <int NPL>
__global__ __launch_bounds__(256) void router_topk_kernel(int64_t T, const uint16_t *X, int H, const float *Wr,
                                                          const float *bias, const double *lg, const uint64_t *bnd,
                                                          int nb, int E, int k, int depth, int32_t *idx, float *wout,
                                                          int32_t *n_fixup) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const double B = 1.01 * gamma_d(depth) * bound_of_slots(bnd + t * nb, nb);
  if (!topk_certified<NPL>(lg + t * E, E, k, B, idx + t * k, wout + t * k)) {
    if (lane == 0 && n_fixup) atomicAdd(n_fixup, 1);
    topk_dd<NPL>(X + t * H, H, Wr, bias, E, k, idx + t * k, wout + t * k, nullptr);
  }
}

__global__ void copy_d2f_kernel(const double *a, int64_t n, float *b) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) b[i] = (float)a[i];
}

// ---------------------------------------------------------------- launchers
template <int NC>
static int launch_logits_nc(hipStream_t st, const uint16_t *X, int64_t T, const float *Wr, const float *bias,
                            int64_t E, const RouterWs &rw, int32_t *n_fixup, int *depth, int *nb) {
  constexpr int H = NC * 256;
  // four tokens per workgroup: more workgroups in flight beat reusing a staged router row
  int tchunk = kTokChunkBytes / (H * 2);
  if (tchunk > 4) tchunk = 4;
  if (tchunk > T) tchunk = (int)T;
  dim3 grid((unsigned)cdiv(E, 4), (unsigned)cdiv(T, tchunk));
  size_t lds = (size_t)tchunk * H * 2;
  TMOE_LAUNCH(TMOE_KERNEL_ROUTER_LOGITS, (router_logits_kernel<NC>), grid, dim3(256), lds, st, X, T, Wr, bias, E,
              tchunk, rw.lg, rw.bnd, n_fixup);
  TMOE_LAUNCHED("router_logits");
  *depth = 4 * NC + 8;
  *nb = (int)grid.x;
  return TMOE_OK;
}

template <int NC, int NPL>
static int launch_router_nc(hipStream_t st, const uint16_t *X, int64_t T, const float *Wr, const float *bias,
                            int64_t E, int k, int32_t *idx, float *w, int32_t *n_fixup, const RouterWs &rw) {
  constexpr int H = NC * 256;
  int depth, nb;
  if (T <= kVectorRouterMaxT) {
    int rc = launch_logits_nc<NC>(st, X, T, Wr, bias, E, rw, n_fixup, &depth, &nb);
    if (rc) return rc;
  } else {
    if (cdiv(T, 16) > 0x7FFFFFFF) return fail(TMOE_E_UNSUPPORTED, "T too large");
    TMOE_LAUNCH(TMOE_KERNEL_ROUTER_LOGITS, (router_mfma_kernel<NC>), dim3((unsigned)cdiv(E, 16), (unsigned)cdiv(T, 16)),
                dim3(256), 0, st, X, T, Wr, bias, (int)E, rw.lg, rw.bnd, n_fixup);
    depth = H + 8;
    nb = (int)cdiv(E, 16);
  }
  TMOE_LAUNCHED("router_logits");
  TMOE_LAUNCH(TMOE_KERNEL_ROUTER_TOPK, (router_topk_kernel<NPL>), dim3((unsigned)cdiv(T, 4)), dim3(256), 0, st, T, X,
              H, Wr, bias, rw.lg, rw.bnd, nb, (int)E, k, depth, idx, w, n_fixup);
  TMOE_LAUNCHED("router_topk");
  return TMOE_OK;
}

// dispatch on H / 256 (NC) and on experts per lane (NPL: E <= 256 -> 4, else 16)
#define TMOE_ROUTER_DISPATCH(FN, ...)                                                      \
  do {                                                                                     \
    const bool small_e = E <= 256;                                                         \
    switch (H / 256) {                                                                     \
      case 1: return small_e ? FN<1, 4>(__VA_ARGS__) : FN<1, 16>(__VA_ARGS__);             \
      case 2: return small_e ? FN<2, 4>(__VA_ARGS__) : FN<2, 16>(__VA_ARGS__);             \
      case 4: return small_e ? FN<4, 4>(__VA_ARGS__) : FN<4, 16>(__VA_ARGS__);             \
      case 8: return small_e ? FN<8, 4>(__VA_ARGS__) : FN<8, 16>(__VA_ARGS__);             \
      case 16: return small_e ? FN<16, 4>(__VA_ARGS__) : FN<16, 16>(__VA_ARGS__);          \
      default: return fail(TMOE_E_UNSUPPORTED, "router hidden size must be 256, 512, 1024, 2048 or 4096"); \
    }                                                                                      \
  } while (0)

int launch_router_logits(hipStream_t st, const uint16_t *X, int64_t T, int64_t H, const float *Wr, const float *bias,
                         int64_t E, const RouterWs &rw, int *depth, int *nb) {
  switch (H / 256) {
    case 1: return launch_logits_nc<1>(st, X, T, Wr, bias, E, rw, nullptr, depth, nb);
    case 2: return launch_logits_nc<2>(st, X, T, Wr, bias, E, rw, nullptr, depth, nb);
    case 4: return launch_logits_nc<4>(st, X, T, Wr, bias, E, rw, nullptr, depth, nb);
    case 8: return launch_logits_nc<8>(st, X, T, Wr, bias, E, rw, nullptr, depth, nb);
    case 16: return launch_logits_nc<16>(st, X, T, Wr, bias, E, rw, nullptr, depth, nb);
    default: return fail(TMOE_E_UNSUPPORTED, "router hidden size must be 256, 512, 1024, 2048 or 4096");
  }
}

int launch_router(hipStream_t st, const uint16_t *X, int64_t T, int64_t H, const float *Wr, const float *bias,
                  int64_t E, int k, int32_t *idx, float *w, float *logits_out, int32_t *n_fixup, const RouterWs &rw) {
  if (T > 0x7FFFFFFF / 4) return fail(TMOE_E_UNSUPPORTED, "T too large");
  int rc = [&]() -> int { TMOE_ROUTER_DISPATCH(launch_router_nc, st, X, T, Wr, bias, E, k, idx, w, n_fixup, rw); }();
  if (rc || !logits_out) return rc;
  hipLaunchKernelGGL(copy_d2f_kernel, dim3((unsigned)cdiv(T * E, 256)), dim3(256), 0, st, rw.lg, T * E, logits_out);
  TMOE_LAUNCHED("logits_copy");
  return TMOE_OK;
}

}  // namespace tmoe
