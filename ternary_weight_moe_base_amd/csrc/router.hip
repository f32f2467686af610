// Full-precision router with a certified top-k.
//
// The router of each layer stays in full precision and selects 8 of 256
// experts from its logits (ai.thesatyajit.com, "The claim, verified from the
// bytes"; codeinsider.com.br, "256 experts, 8 ativos"). The selection must
// equal that of the exact logits, so the fp32 pass carries a rigorous error
// bound and tokens whose top-(k+1) ranking it cannot separate are recomputed in
// fp64 with exact products.
#include "common.h"

namespace tmoe {

static constexpr int kTokChunkBytes = 65536;  // LDS bytes of bf16 activations per workgroup

size_t router_ws_bytes(int64_t T, int64_t E) {
  size_t o = 0;
  o = align_up(o + E * 4, 256);      // wl1
  o = align_up(o + T * E * 4, 256);  // logits
  o = align_up(o + 4, 256);          // fix_count
  o = align_up(o + T * 4, 256);      // fix_list
  return o;
}

RouterWs router_ws_carve(void *ws, int64_t T, int64_t E) {
  char *b = (char *)ws;
  RouterWs r;
  size_t o = 0;
  r.wl1 = (float *)(b + o);
  o = align_up(o + E * 4, 256);
  r.logits = (float *)(b + o);
  o = align_up(o + T * E * 4, 256);
  r.fix_count = (int32_t *)(b + o);
  o = align_up(o + 4, 256);
  r.fix_list = (int32_t *)(b + o);
  return r;
}

__device__ inline float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ inline double wave_sum_d(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// ------------------------------------------------------------ fp32 logits
// Workgroup = 4 wavefronts = 4 experts; grid.y walks token chunks staged in
// LDS. Each lane keeps 4*NC router weights in registers (elements
// c*256 + 4*lane + 0..3) and runs one FMA chain of 4*NC terms per logit, then
// a 6-level butterfly: every product is rounded at most 4*NC + 6 times.
template <int NC>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t *X, int64_t T, const float *Wr,
                                                            const float *bias, int64_t E, int tchunk, float *logits,
                                                            float *wl1, int32_t *fix_count) {
  extern __shared__ __align__(16) uint16_t xs[];  // [tchunk][H]
  constexpr int H = NC * 256;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t e = (int64_t)blockIdx.x * 4 + wave;
  const int64_t t0 = (int64_t)blockIdx.y * tchunk;
  const int nt = (int)min<int64_t>(tchunk, T - t0);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *fix_count = 0;
  // stage activations (16-byte copies)
  const int vec_per_row = H / 8;
  for (int i = threadIdx.x; i < nt * vec_per_row; i += 256) {
    int n = i / vec_per_row, c = i % vec_per_row;
    reinterpret_cast<uint4 *>(xs + (size_t)n * H)[c] = reinterpret_cast<const uint4 *>(X + (t0 + n) * H)[c];
  }
  __syncthreads();
  if (e >= E) return;
  float4 w[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) w[c] = reinterpret_cast<const float4 *>(Wr + e * H)[c * 64 + lane];
  if (blockIdx.y == 0) {
    float a = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) a += fabsf(w[c].x) + fabsf(w[c].y) + fabsf(w[c].z) + fabsf(w[c].w);
    a = wave_sum(a);
    if (lane == 0) wl1[e] = a;
  }
  const float b = bias ? bias[e] : 0.f;
  for (int n = 0; n < nt; ++n) {
    const uint2 *xr = reinterpret_cast<const uint2 *>(xs + (size_t)n * H);
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint2 xv = xr[c * 64 + lane];
      acc = fmaf(w[c].x, __uint_as_float(xv.x << 16), acc);
      acc = fmaf(w[c].y, __uint_as_float(xv.x & 0xFFFF0000u), acc);
      acc = fmaf(w[c].z, __uint_as_float(xv.y << 16), acc);
      acc = fmaf(w[c].w, __uint_as_float(xv.y & 0xFFFF0000u), acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) logits[(t0 + n) * E + e] = acc + b;
  }
}

// Wave-wide selection of the best (value, index): larger value, then lower index.
__device__ inline void wave_argmax(float &v, int &i) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    float ov = __shfl_xor(v, m, 64);
    int oi = __shfl_xor(i, m, 64);
    if (ov > v || (ov == v && oi < i)) {
      v = ov;
      i = oi;
    }
  }
}
__device__ inline void wave_argmax_d(double &v, int &i) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    double ov = __shfl_xor(v, m, 64);
    int oi = __shfl_xor(i, m, 64);
    if (ov > v || (ov == v && oi < i)) {
      v = ov;
      i = oi;
    }
  }
}

// ---------------------------------------------------- certified top-k (fp32)
// One wavefront per token. Error bound (Higham, "Accuracy and Stability of
// Numerical Algorithms", recursive summation with FMA): every logit satisfies
// |fl(l) - l| <= gamma_d * (||x||_inf * ||w_e||_1 + |b_e|), gamma_d = d u / (1 - d u),
// u = 2^-24, d = 4*NC + 8 (chain + butterfly + bias + margin). With the largest
// ||w_e||_1 and |b_e| this is one bound B for the whole token; the ranking of
// the top k+1 is certified when all adjacent gaps exceed 2B.
__global__ __launch_bounds__(256) void router_topk_kernel(const uint16_t *X, int64_t T, int H, const float *logits,
                                                          const float *wl1, const float *bias, int E, int k,
                                                          int depth, int32_t *idx, float *wout, int32_t *fix_count,
                                                          int32_t *fix_list) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float xi = 0.f;
  for (int i = lane; i < H; i += 64) xi = fmaxf(xi, fabsf(bf16f(X[t * H + i])));
  xi = wave_max(xi);
  float wm = 0.f, bm = 0.f;
  for (int e = lane; e < E; e += 64) {
    wm = fmaxf(wm, wl1[e]);
    if (bias) bm = fmaxf(bm, fabsf(bias[e]));
  }
  wm = wave_max(wm);
  bm = wave_max(bm);
  const double u = 0x1p-24;
  const double gam = depth * u / (1.0 - depth * u);
  const float B = (float)(1.01 * gam * ((double)xi * (double)wm * (1.0 + 1e-3) + (double)bm));
  // logits of this lane: experts lane + 64*j
  float lv[16];
  uint32_t taken = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    int e = lane + 64 * j;
    lv[j] = e < E ? logits[t * E + e] : -INFINITY;
    if (e >= E) taken |= 1u << j;
  }
  const int m = min(k + 1, E);
  // ranks 0..m-1 in order; lane r keeps rank r (value, index)
  float prev = 0.f, myv = -INFINITY, v0 = 0.f;
  int myi = 0;
  bool ok = true;
  for (int r = 0; r < m; ++r) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF, bj = -1;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (taken & (1u << j)) continue;
      if (bj < 0 || lv[j] > bv) {  // within a lane, the expert index grows with j
        bv = lv[j];
        bi = lane + 64 * j;
        bj = j;
      }
    }
    wave_argmax(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (r == 0) v0 = bv;
    else ok = ok && (prev - bv > 2.f * B);
    prev = bv;
    if (r == lane) {
      myv = bv;
      myi = bi;
    }
  }
  if (!ok) {
    if (lane == 0) {
      int slot = atomicAdd(fix_count, 1);
      fix_list[slot] = (int32_t)t;
    }
    return;
  }
  const float p = lane < k ? expf(myv - v0) : 0.f;
  const float den = wave_sum(p);
  if (lane < k) {
    idx[t * k + lane] = myi;
    wout[t * k + lane] = p / den;
  }
}

// --------------------------------------------------------- fp64 recompute
// One workgroup per token listed by the certified pass. Products bf16 * fp32
// are exact in fp64; every expert's sum uses the same lane-strided chain and
// butterfly, so identical router rows give bit-identical logits (ties then go
// to the lower index, as for exact logits).
__global__ __launch_bounds__(256) void router_fixup_kernel(const uint16_t *X, int H, const float *Wr,
                                                           const float *bias, int E, int k, const int32_t *fix_count,
                                                           const int32_t *fix_list, int32_t *idx, float *wout,
                                                           int32_t *n_fixup) {
  __shared__ double lg[1024];
  const int nfix = *fix_count;
  if (blockIdx.x == 0 && threadIdx.x == 0 && n_fixup) *n_fixup = nfix;
  if ((int)blockIdx.x >= nfix) return;
  const int64_t t = fix_list[blockIdx.x];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t *x = X + t * H;
  for (int e = wave; e < E; e += 4) {
    const float *w = Wr + (int64_t)e * H;
    double acc = 0.0;
    for (int i = lane; i < H; i += 64) acc += (double)bf16f(x[i]) * (double)w[i];
    acc = wave_sum_d(acc);
    if (lane == 0) lg[e] = acc + (bias ? (double)bias[e] : 0.0);
  }
  __syncthreads();
  if (wave != 0) return;
  double lv[16];
  uint32_t taken = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    int e = lane + 64 * j;
    lv[j] = e < E ? lg[e] : -INFINITY;
    if (e >= E) taken |= 1u << j;
  }
  double myv = -INFINITY, v0 = 0.0;
  int myi = 0;
  for (int r = 0; r < k; ++r) {
    double bv = -INFINITY;
    int bi = 0x7FFFFFFF, bj = -1;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (taken & (1u << j)) continue;
      if (bj < 0 || lv[j] > bv) {
        bv = lv[j];
        bi = lane + 64 * j;
        bj = j;
      }
    }
    wave_argmax_d(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (r == 0) v0 = bv;
    if (r == lane) {
      myv = bv;
      myi = bi;
    }
  }
  const double p = lane < k ? exp(myv - v0) : 0.0;
  const double den = wave_sum_d(p);
  if (lane < k) {
    idx[t * k + lane] = myi;
    wout[t * k + lane] = (float)(p / den);
  }
}

template <int NC>
static void launch_logits(hipStream_t st, const uint16_t *X, int64_t T, const float *Wr, const float *bias,
                          int64_t E, float *logits, float *wl1, int32_t *fix_count) {
  const int H = NC * 256;
  int tchunk = kTokChunkBytes / (H * 2);
  if (tchunk > T) tchunk = (int)T;
  dim3 grid((unsigned)cdiv(E, 4), (unsigned)cdiv(T, tchunk));
  size_t lds = (size_t)tchunk * H * 2;
  hipLaunchKernelGGL(router_logits_kernel<NC>, grid, dim3(256), lds, st, X, T, Wr, bias, E, tchunk, logits, wl1,
                     fix_count);
}

int launch_router(hipStream_t st, const uint16_t *X, int64_t T, int64_t H, const float *Wr, const float *bias,
                  int64_t E, int k, int32_t *idx, float *w, float *logits_out, int32_t *n_fixup, const RouterWs &rw) {
  if (H % 256 != 0 || H > 4096) return fail(TMOE_E_UNSUPPORTED, "router needs H %% 256 == 0 and H <= 4096");
  if (T > 0x7FFFFFFF / 4) return fail(TMOE_E_UNSUPPORTED, "T too large");
  float *logits = logits_out ? logits_out : rw.logits;
  switch (H / 256) {
#define CASE(n) \
  case n: launch_logits<n>(st, X, T, Wr, bias, E, logits, rw.wl1, rw.fix_count); break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
    CASE(9) CASE(10) CASE(11) CASE(12) CASE(13) CASE(14) CASE(15) CASE(16)
#undef CASE
  }
  TMOE_LAUNCHED("router_logits");
  const int depth = 4 * (int)(H / 256) + 8;
  hipLaunchKernelGGL(router_topk_kernel, dim3((unsigned)cdiv(T, 4)), dim3(256), 0, st, X, T, (int)H, logits, rw.wl1,
                     bias, (int)E, k, depth, idx, w, rw.fix_count, rw.fix_list);
  TMOE_LAUNCHED("router_topk");
  hipLaunchKernelGGL(router_fixup_kernel, dim3((unsigned)T), dim3(256), 0, st, X, (int)H, Wr, bias, (int)E, k,
                     rw.fix_count, rw.fix_list, idx, w, n_fixup);
  TMOE_LAUNCHED("router_fixup");
  return TMOE_OK;
}

}  // namespace tmoe
