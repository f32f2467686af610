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
static constexpr int kVectorRouterMaxT = 64;  // up to 64 tokens the VALU kernel beats the matrix cores
// From this many tokens on, a call that does not return the logits picks
// candidates on the bf16 matrix cores (below it the fp64 matrix-core logits
// are faster)
static constexpr int kBf16RouterMinT = 1024;
static constexpr int kRgMaxSK = 4;  // input slices of the logits GEMM

size_t router_ws_bytes(int64_t T, int64_t E, int64_t H) {
  size_t o = 0;
  o = align_up(o + T * cdiv(E, 4) * 8, 256);  // bnd
  o = align_up(o + T * E * 8, 256);  // lg
  if (T >= kBf16RouterMinT) {
    o = align_up(o + (size_t)2 * E * H * 2, 256);  // bf16 parts w1, w2 of the router rows
    o = align_up(o + (size_t)2 * cdiv(E, 4) * 8, 256);       // norm / bias maxima per split workgroup
    o = align_up(o + (size_t)E * 8, 256);                    // row norms
    o = align_up(o + (size_t)kRgMaxSK * T * E * 4, 256);     // fp32 slice sums of the candidate logits
  }
  return o;
}

RouterWs router_ws_carve(void *ws, int64_t T, int64_t E, int64_t H) {
  char *b = (char *)ws;
  RouterWs r;
  size_t o = 0;
  r.bnd = (uint64_t *)(b + o);
  o = align_up(o + T * cdiv(E, 4) * 8, 256);
  r.lg = (double *)(b + o);
  o = align_up(o + T * E * 8, 256);
  r.parts = nullptr;
  r.wmax = nullptr;
  r.wnorm = nullptr;
  r.part = nullptr;
  if (T >= kBf16RouterMinT) {
    r.parts = (uint16_t *)(b + o);
    o = align_up(o + (size_t)2 * E * H * 2, 256);
    r.wmax = (uint64_t *)(b + o);
    o = align_up(o + (size_t)2 * cdiv(E, 4) * 8, 256);
    r.wnorm = (double *)(b + o);
    o = align_up(o + (size_t)E * 8, 256);
    r.part = (float *)(b + o);
  }
  return r;
}

// ------------------------------------------------------------ fp64 logits
// One token's chains over this lane's inputs (exact bf16 x fp32 products in
// fp64): the logit sum and the sum of |x w| for the bound.
// Two chains of 2 NC products each (inputs of even and odd c), then their sum:
// no element passes more than 2 NC + 1 roundings here, within the 4 NC that
// the bound's depth counts for this part.
template <int NC>
__device__ __forceinline__ void logit_chains(const uint2 *xr, const double (&w)[4 * NC], int lane, double &acc,
                                             double &aab) {
  double a2[2] = {0.0, 0.0}, b2[2] = {0.0, 0.0};
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    uint2 xv = xr[c * 64 + lane];
    const double x0 = __uint_as_float(xv.x << 16), x1 = __uint_as_float(xv.x & 0xFFFF0000u);
    const double x2 = __uint_as_float(xv.y << 16), x3 = __uint_as_float(xv.y & 0xFFFF0000u);
    double &a = a2[c & 1], &b = b2[c & 1];
    a = fma(w[4 * c], x0, a);
    a = fma(w[4 * c + 1], x1, a);
    a = fma(w[4 * c + 2], x2, a);
    a = fma(w[4 * c + 3], x3, a);
    b = fma(fabs(w[4 * c]), fabs(x0), b);
    b = fma(fabs(w[4 * c + 1]), fabs(x1), b);
    b = fma(fabs(w[4 * c + 2]), fabs(x2), b);
    b = fma(fabs(w[4 * c + 3]), fabs(x3), b);
  }
  acc = a2[0] + a2[1];
  aab = b2[0] + b2[1];
}

// Each lane keeps 4*NC router weights (elements c*256 + 4*lane + 0..3, loaded
// by the caller as wv[c]) as fp64 and sums its 4*NC exact products per logit
// in two FMA chains (logit_chains), then a 6-level DPP butterfly: depth at most
// 4*NC + 6, plus 1 for the bias (bv: the caller's bias value, used when bias
// is not null); the bound counts 4*NC + 8. The same chains accumulate
// A = sum |x w| for the bound. Four tokens go together (sixteen independent
// chains) when the chunk holds them. Results for token n go to lgs[n*4 + wave]
// and abs_s[n*4 + wave] (LDS).
template <int NC>
__device__ inline void logits_rows(const uint16_t *xs, int nt, const float4 (&wv)[NC], const float *bias, float bv,
                                   int64_t e, int E, double *lgs, double *abs_s) {
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
    const float4 v = wv[c];
    w[4 * c] = v.x;
    w[4 * c + 1] = v.y;
    w[4 * c + 2] = v.z;
    w[4 * c + 3] = v.w;
  }
  const double b = bias ? (double)bv : 0.0;
  int n = 0;
  for (; n + 4 <= nt; n += 4) {
    double acc[4], aab[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      logit_chains<NC>(reinterpret_cast<const uint2 *>(xs + (size_t)(n + u) * H), w, lane, acc[u], aab[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[u] = wave_sum_dpp(acc[u]);
      aab[u] = wave_sum_dpp(aab[u]);
    }
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        lgs[(n + u) * 4 + wave] = acc[u] + b;
        abs_s[(n + u) * 4 + wave] = aab[u] + fabs(b);
      }
    }
  }
  for (; n < nt; ++n) {
    double acc, aab;
    logit_chains<NC>(reinterpret_cast<const uint2 *>(xs + (size_t)n * H), w, lane, acc, aab);
    acc = wave_sum_dpp(acc);
    aab = wave_sum_dpp(aab);
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
  // this wavefront's router row first, so its fetch overlaps the activation
  // staging (rows past E read row E - 1 and are not used: no branch around the
  // loads, which would make the compiler wait for each one)
  const int64_t e = e0 + (threadIdx.x >> 6);
  const float4 *wrow = reinterpret_cast<const float4 *>(Wr + min<int64_t>(e, E - 1) * (NC * 256));
  float4 wv[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) wv[c] = wrow[c * 64 + (threadIdx.x & 63)];
  const float bv = (bias ? bias : Wr)[min<int64_t>(e, E - 1)];  // unused without a bias
  stage_x(xs, X, t0, nt, NC * 256);
  __syncthreads();
  logits_rows<NC>(xs, nt, wv, bias, bv, e, (int)E, lgs, abs_s);
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

// ------------------------------------------------- bf16 matrix-core logits
// With many tokens the logits are first formed on the bf16 matrix cores, only
// to pick each token's candidates; the candidates are then recomputed in fp64
// by the top-k kernel, whose ranking and softmax use only those values. Each
// fp32 router weight is split into bf16 parts w = w1 + w2 + w3 (each rounding
// keeps the next 8 of its 24 significant bits; |w3| <= 2^-16 |w|); the
// candidate logits use w1 + w2 (a bf16 activation times a bf16 part is exact
// in fp32), and the bound counts the w3 left out.
//
// Split pass: wavefront w of workgroup b takes router row e = 4b + w: its
// parts w1, w2 go to parts[q][e][*], its norm |w_e|_2 (fp64 sum of exact
// squares) to wnorm[e], and the workgroup's largest row norm and largest
// |b_e| to slots wmax[b], wmax[nslots + b] (fp64 bits). Also clears the
// fix-up counter.
template <int NC>
__global__ __launch_bounds__(256) void router_split_kernel(const float *Wr, const float *bias, int E,
                                                           uint16_t *parts, uint64_t *wmax, int nslots,
                                                           double *wnorm, int32_t *n_fixup) {
  constexpr int H = NC * 256;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x * 4 + wave;
  __shared__ double nw[4], nb[4];
  if (blockIdx.x == 0 && threadIdx.x == 0 && n_fixup) *n_fixup = 0;
  // |b_e| fetched first and unconditionally (a valid address either way)
  const float bv = (bias ? bias : Wr)[min(e, E - 1)];
  double s2 = 0.0;
  if (e < E) {
    const size_t plane = (size_t)E * H;
    // the row's NC loads are all in flight before the first conversion
    float4 rv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) rv[c] = *reinterpret_cast<const float4 *>(Wr + (size_t)e * H + c * 256 + lane * 4);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int i = c * 256 + lane * 4;
      const float4 v = rv[c];
      const float f[4] = {v.x, v.y, v.z, v.w};
      uint32_t pw[2][2] = {};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t h = f32_to_bf16_rne(f[j]);
        const uint32_t m = f32_to_bf16_rne(f[j] - bf16f((uint16_t)h));
        const int sh = 16 * (j & 1);
        pw[0][j >> 1] |= h << sh;
        pw[1][j >> 1] |= m << sh;
        s2 = fma((double)f[j], (double)f[j], s2);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q)
        *reinterpret_cast<uint2 *>(parts + q * plane + (size_t)e * H + i) = make_uint2(pw[q][0], pw[q][1]);
    }
  }
  s2 = wave_sum_dpp(s2);
  if (lane == 0) {
    nw[wave] = sqrt(s2);
    if (e < E) wnorm[e] = nw[wave];
    nb[wave] = (e < E && bias) ? fabs((double)bv) : 0.0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    wmax[blockIdx.x] = dbits(fmax(fmax(nw[0], nw[1]), fmax(nw[2], nw[3])));
    wmax[nslots + blockIdx.x] = dbits(fmax(fmax(nb[0], nb[1]), fmax(nb[2], nb[3])));
  }
}

// Logits pass, a bf16 GEMM: workgroup = 4 wavefronts over a tile of 128
// router rows x 128 tokens and one of SK slices of the inputs; wavefront
// (we, wt) takes rows e0 + 64 we .. + 63 (4 row tiles of 16) and tokens
// t0 + 64 wt .. + 63 (4 token tiles). Each K step of 32 inputs (parts w1, w2
// of the 128 rows and the 128 token rows: 384 rows of 64 B) goes from memory
// straight into LDS by buffer loads (no registers), kRgStages - 1 steps ahead
// of its products. A staged row holds its four 16-byte chunks in the order
// c ^ ((row >> 2) & 3), so the 16 lanes that read one chunk of 16 consecutive
// rows hit 16 distinct groups of four banks. One barrier per step: past it
// every wavefront's loads of the step have landed and every wavefront has
// finished its reads of the previous step, whose buffer the loads issued next
// refill. Per step a wavefront runs 4 x 4 tiles x 2 parts products, w1 and w2
// of a tile into one fp32 accumulator. part[sk][t][e] = the slice's sum
// (fp32). Rows past E and tokens past T read a valid row and are not stored.
constexpr int kRgStages = 6;            // staged K steps (kRgStages - 1 in flight ahead)
constexpr int kRgStage = 384 * 64;      // bytes per staged step
constexpr int kRgLoads = 384 * 4 / 256;  // 16-byte loads per thread per step (6)

// s_waitcnt vmcnt(n) for n = kRgLoads * m, m = 0 .. kRgStages - 2
__device__ __forceinline__ void rg_wait(int m) {
  switch (m) {
    case 0: TMOE_WAIT_VM(0); break;
    case 1: TMOE_WAIT_VM(kRgLoads); break;
    case 2: TMOE_WAIT_VM(2 * kRgLoads); break;
    case 3: TMOE_WAIT_VM(3 * kRgLoads); break;
    default: TMOE_WAIT_VM(4 * kRgLoads); break;
  }
}
static_assert(kRgStages - 2 <= 4, "rg_wait covers up to four later steps");

template <int SK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void router_gemm_kernel(const uint16_t *X, int64_t T, const uint16_t *parts, int E,
                                                          int H, int neb, float *part) {
  extern __shared__ __align__(16) char lds[];  // [kRgStages][384 rows][64 B]
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int we = wave & 1, wt = wave >> 1;
  const int sk = blockIdx.x % SK, tile = blockIdx.x / SK;
  const int eb = tile % neb, tb = tile / neb;
  const int e0 = eb * 128;
  const int64_t t0 = (int64_t)tb * 128;
  const int nstep = H / 32 / SK;
  const int kbase = sk * nstep * 32;
  // load instruction u of this wavefront fills LDS chunks 64 (kRgLoads wave + u) + lane of a step:
  // staged row (chunks / 4) < 256 are router rows (w1: 0..127, w2: 128..255), the rest token rows
  const int ntok = (int)min<int64_t>(128, T - t0);
  const __amdgpu_buffer_rsrc_t rp =
      __builtin_amdgcn_make_buffer_rsrc((void *)parts, (short)0, (int)((int64_t)2 * E * H * 2), kBufWord3);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void *)(X + t0 * H), (short)0, ntok * H * 2, kBufWord3);
  int voff[kRgLoads];
#pragma unroll
  for (int u = 0; u < kRgLoads; ++u) {
    const int L = (kRgLoads * wave + u) * 64 + lane, row = L >> 2;
    const int c = (L & 3) ^ ((row >> 2) & 3);  // the input chunk this lane stages
    if (row < 256) {
      const int q = row >> 7, e = min(e0 + (row & 127), E - 1);
      voff[u] = ((q * E + e) * H + kbase + 8 * c) * 2;
    } else {
      voff[u] = (min(row - 256, ntok - 1) * H + kbase + 8 * c) * 2;
    }
  }
  // instructions u with (kRgLoads wave + u) < 16 stage router rows (wave-uniform)
#define RG_ISSUE(S)                                                                                            \
  do {                                                                                                         \
    char *b_ = lds + ((S) % kRgStages) * kRgStage;                                                             \
    _Pragma("unroll") for (int u = 0; u < kRgLoads; ++u) {                                                     \
      __attribute__((address_space(3))) void *d_ = (__attribute__((address_space(3))) void *)(b_ + (kRgLoads * wave + u) * 1024); \
      if (kRgLoads * wave + u < 16)                                                                            \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, d_, 16, voff[u], 64 * (S), 0, 0);                        \
      else                                                                                                     \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, d_, 16, voff[u], 64 * (S), 0, 0);                        \
    }                                                                                                          \
  } while (0)
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int r16 = lane & 15, kq = lane >> 4;
  const int rd = r16 * 64 + ((kq ^ ((r16 >> 2) & 3)) << 4);  // this lane's chunk in a group of 16 rows
#pragma unroll
  for (int s = 0; s < kRgStages - 1; ++s)
    if (s < nstep) RG_ISSUE(s);
#pragma unroll 1
  for (int s = 0; s < nstep; ++s) {
    rg_wait(min(kRgStages - 2, nstep - 1 - s));
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wavefront's reads of step s - 1 are done
    __builtin_amdgcn_s_barrier();
    if (s + kRgStages - 1 < nstep) RG_ISSUE(s + kRgStages - 1);
    const char *b = lds + (s % kRgStages) * kRgStage + rd;
    u32x4 av[4][2], bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 2; ++q) av[i][q] = lds16(b + (q * 128 + we * 64 + 16 * i) * 64);
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = lds16(b + (256 + wt * 64 + 16 * j) * 64);
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[i][q]),
                                                              __builtin_bit_cast(bf16x8, bv[j]), acc[i][j], 0, 0, 0);
  }
#undef RG_ISSUE
  // lane: token t0 + 64 wt + 16 j + r16, rows e0 + 64 we + 16 i + 4 kq .. + 3
  float *out = part + (size_t)sk * T * E;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t t = t0 + wt * 64 + 16 * j + r16;
    if (t >= T) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + we * 64 + 16 * i + 4 * kq;
      if (e + 3 < E && (E & 3) == 0) {
        *reinterpret_cast<float4 *>(out + t * E + e) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (e + v < E) out[t * E + e + v] = acc[i][j][v];
      }
    }
  }
}

// Certified top-k from the matrix-core logits l~ (error <= B1 for every
// expert), one wavefront per token:
//  1. the (k+1)-th largest of 32-bit keys (l~ rounded to fp32, order-
//     preserving, low IB bits replaced by the expert index) gives a bucket
//     whose lowest value f_low is at most the (k+1)-th largest l~ up to the
//     fp32 rounding; every expert with l~ >= thr = f_low - 2^-22 |f_low| - 2 B1
//     is a candidate (the true top k+1 are among them: any other has a true
//     logit below c - B1, under all k+1 of those with l~ >= c, the (k+1)-th
//     largest l~). The list goes to LDS in ascending expert order.
//  2. each candidate is recomputed in fp64 (exact products, an FMA chain of
//     4 NC per lane, a DPP butterfly of depth 6), kRfBatch at a time with all
//     their loads in flight; lane i keeps candidate i.
//  3. each candidate's rank is counted (larger value first, equal values to
//     the lower expert); the top k+1 adjacent gaps are certified against
//     2 B2, B2 = 1.01 gamma_d max over the candidates of |x|_2 |w_e|_2 +
//     |b_e|, and idx and the softmax over the k (fp64 values) are written.
// A token with more than 64 candidates, or not certified, is recomputed in
// double-double (counted in *n_fixup).
constexpr int kRfBatch = 2;  // rows in flight per batch (three waves per SIMD fit)

template <int NPL, int NC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void router_topk_refine_kernel(int64_t T, const uint16_t *X, const float *Wr,
                                                                 const float *bias, const float *part, int SK,
                                                                 const uint64_t *wmax, int nslots,
                                                                 const double *wnorm, int E, int k, double gfac,
                                                                 double babs, int32_t *idx, float *wout,
                                                                 int32_t *n_fixup) {
  constexpr int H = NC * 256;
  constexpr int IB = NPL * 64 <= 256 ? 8 : 10;  // index bits of a key
  __shared__ int32_t cand[4][64];
  __shared__ double rank_v[4][17];
  __shared__ int32_t rank_e[4][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;
  const uint16_t *x = X + t * H;
  // every load the first step needs is issued before the first wait (no
  // branches around them: indices are clamped, extra values unused): the
  // token's inputs, the slots of row-norm and bias maxima, the SK partial sums
  uint2 xp[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) xp[c] = reinterpret_cast<const uint2 *>(x)[c * 64 + lane];
  uint64_t wmv[kRouterMaxSlots / 64], bmv[kRouterMaxSlots / 64];
#pragma unroll
  for (int u = 0; u < kRouterMaxSlots / 64; ++u) {
    const int j = min(lane + 64 * u, nslots - 1);
    wmv[u] = wmax[j];
    bmv[u] = wmax[nslots + j];
  }
  float pv[kRgMaxSK][NPL];
#pragma unroll
  for (int q = 0; q < kRgMaxSK; ++q) {
    const float *pr = part + ((size_t)min(q, SK - 1) * T + t) * E;
#pragma unroll
    for (int j = 0; j < NPL; ++j) pv[q][j] = pr[min(lane * NPL + j, E - 1)];
  }
  double s2 = 0.0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const double q[4] = {__uint_as_float(xp[c].x << 16), __uint_as_float(xp[c].x & 0xFFFF0000u),
                         __uint_as_float(xp[c].y << 16), __uint_as_float(xp[c].y & 0xFFFF0000u)};
#pragma unroll
    for (int i = 0; i < 4; ++i) s2 = fma(q[i], q[i], s2);
  }
  const double nx = 1.01 * sqrt(wave_sum_dpp(s2));  // |x_t|_2 with a 1% margin
  uint64_t wm = 0, bm = 0;
#pragma unroll
  for (int u = 0; u < kRouterMaxSlots / 64; ++u) {
    wm = wm > wmv[u] ? wm : wmv[u];
    bm = bm > bmv[u] ? bm : bmv[u];
  }
  const double B1 = gfac * (nx * __longlong_as_double((long long)wave_max_u64(wm)) +
                            __longlong_as_double((long long)wave_max_u64(bm))) + babs;

  // ---- 1. candidates (the slice sums added in slice order, as before)
  double v[NPL];
  uint32_t key[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) v[j] = 0.0;
#pragma unroll
  for (int q = 0; q < kRgMaxSK; ++q)
#pragma unroll
    for (int j = 0; j < NPL; ++j) v[j] += q < SK ? (double)pv[q][j] : 0.0;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane * NPL + j;
    if (e < E && bias) v[j] += (double)bias[e];
    uint32_t u = __float_as_uint((float)v[j]);
    if (u == 0x80000000u) u = 0u;
    const uint32_t o = (u >> 31) ? ~u : (u | 0x80000000u);
    key[j] = e < E ? (((o >> IB) << IB) | (uint32_t)(E - 1 - e)) : 0u;
  }
#pragma unroll
  for (int pass = 0; pass < NPL; ++pass)
#pragma unroll
    for (int j = pass & 1; j + 1 < NPL; j += 2)
      if (key[j] < key[j + 1]) {
        const uint32_t tk = key[j];
        key[j] = key[j + 1];
        key[j + 1] = tk;
      }
  const int m = min(k + 1, E);
  uint32_t mx = 0u;
  for (int r = 0; r < m; ++r) {
    mx = wave_max_u32(key[0]);
    if (key[0] == mx) {
#pragma unroll
      for (int j = 0; j + 1 < NPL; ++j) key[j] = key[j + 1];
      key[NPL - 1] = 0u;
    }
  }
  const uint32_t ob = (mx >> IB) << IB;  // the (k+1)-th key's bucket, lowest value
  const float flow = __uint_as_float((ob >> 31) ? (ob & 0x7FFFFFFFu) : ~ob);
  const double thr = (double)flow - 0x1p-22 * fabs((double)flow) - 2.0 * B1;
  int mine = 0;
#pragma unroll
  for (int j = 0; j < NPL; ++j) mine += (lane * NPL + j < E && v[j] >= thr) ? 1 : 0;
  int incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  const int nc = __builtin_amdgcn_readlane(incl, 63);
  bool ok = nc <= 64 && nc >= m;
  if (ok) {
    int at = incl - mine;
#pragma unroll
    for (int j = 0; j < NPL; ++j)
      if (lane * NPL + j < E && v[j] >= thr) cand[wave][at++] = lane * NPL + j;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();

    // ---- 2. fp64 values of the candidates. Lane i fetches candidate i's bias
    // and row norm now, in flight with the first batch of rows (loaded where
    // they are used, they would cost a round trip per candidate).
    const int mye = cand[wave][min(lane, nc - 1)];
    const double cb = bias ? (double)bias[mye] : 0.0;
    const double cw = wnorm[mye];
    double myv = 0.0;
    for (int i0 = 0; i0 < nc; i0 += kRfBatch) {
      int eb[kRfBatch];
      float4 q[kRfBatch][NC];
#pragma unroll
      for (int u = 0; u < kRfBatch; ++u) {
        eb[u] = cand[wave][min(i0 + u, nc - 1)];
        const float4 *wr = reinterpret_cast<const float4 *>(Wr + (size_t)eb[u] * H);
#pragma unroll
        for (int c = 0; c < NC; ++c) q[u][c] = wr[c * 64 + lane];
      }
      double acc[kRfBatch];
#pragma unroll
      for (int u = 0; u < kRfBatch; ++u) acc[u] = 0.0;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const double x0 = __uint_as_float(xp[c].x << 16), x1 = __uint_as_float(xp[c].x & 0xFFFF0000u);
        const double x2 = __uint_as_float(xp[c].y << 16), x3 = __uint_as_float(xp[c].y & 0xFFFF0000u);
#pragma unroll
        for (int u = 0; u < kRfBatch; ++u) {
          acc[u] = fma((double)q[u][c].x, x0, acc[u]);
          acc[u] = fma((double)q[u][c].y, x1, acc[u]);
          acc[u] = fma((double)q[u][c].z, x2, acc[u]);
          acc[u] = fma((double)q[u][c].w, x3, acc[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < kRfBatch; ++u) {
        const double sum = wave_sum_dpp(acc[u]);
        myv = lane == i0 + u ? sum + cb : myv;
      }
    }
    const double myb = lane < nc ? nx * cw + fabs(cb) : 0.0;
    // B2 over the candidates; chain 4 NC, butterfly 6, bias 1, margin 2
    const double B2 = 1.01 * gamma_d(4 * NC + 9) * __longlong_as_double((long long)wave_max_u64(dbits(myb)));

    // ---- 3. ranks (lane i < nc: larger values first, equal values to the lower expert = lower lane)
    int rank = 0;
    for (int j = 0; j < nc; ++j) {
      const double vj = readlane_d(myv, j);
      rank += (vj > myv || (vj == myv && j < lane)) ? 1 : 0;
    }
    if (lane < nc && rank <= k) {
      rank_v[wave][rank] = myv;
      rank_e[wave][rank] = mye;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
    const int m2 = min(k + 1, nc);
    const double rv = lane < m2 ? rank_v[wave][lane] : 0.0;
    const double nv = lane + 1 < m2 ? rank_v[wave][lane + 1] : 0.0;
    ok = __ballot(lane + 1 < m2 && !(rv - nv > 2.0 * B2)) == 0ull;
    if (ok) {
      const double v0 = readlane_d(rv, 0);
      const double p = lane < k ? exp(rv - v0) : 0.0;
      double den = 0.0;
      for (int r = 0; r < k; ++r) den += readlane_d(p, r);
      if (lane < k) {
        idx[t * k + lane] = rank_e[wave][lane];
        wout[t * k + lane] = (float)(p / den);
      }
    }
  }
  if (!ok) {
    if (lane == 0 && n_fixup) atomicAdd(n_fixup, 1);
    topk_dd<NPL>(x, H, Wr, bias, E, k, idx + t * k, wout + t * k, nullptr);
  }
}

// Bound factor of the matrix-core logits (unit roundoff 2^-24 for fp32, 2^-53
// for fp64; Higham's gamma_n = n u / (1 - n u), which bounds a sum of n + 1
// terms in any order): |l~ - l| <= gfac (|x|_2 max_e |w_e|_2 + max_e |b_e|) +
// babs, with sum_i |x_i w_i| <= |x|_2 |w|_2 (Cauchy-Schwarz). Terms: each of
// the SK slice sums adds 2 x 32 exact products per K step to one fp32 sum
// (at most 66 roundings a step on any path; |w1| + |w2| <= (1 + 2^-7)|w|);
// the w3 left out (|w3| <= 2^-16 |w|); the fp64 sum of the slices and the
// bias; 1% margin for the norms' own rounding. babs covers subnormal parts
// and products the matrix cores may flush.
static void router_bf16_bound(int H, int SK, double *gfac, double *babs) {
  auto g32 = [](double n) { const double u = 0x1p-24; return n * u / (1.0 - n * u); };
  auto g64 = [](double n) { const double u = 0x1p-53; return n * u / (1.0 - n * u); };
  const double steps = H / 32.0 / SK;
  const double t1 = g32(66.0 * steps) * (1.0 + 0x1p-7);
  const double t2 = 0x1p-16;
  const double t3 = g64(SK + 2.0) * (1.0 + 0x1p-7);
  *gfac = 1.01 * (t1 + t2 + t3);
  *babs = (double)H * 0x1p-120;
}

// One wavefront per token: certified top-k from the fp64 logits, else the
// double-double recompute (counted in *n_fixup).
template <int NPL>
__global__ __launch_bounds__(256) void router_topk_kernel(int64_t T, const uint16_t *X, int H, const float *Wr,
                                                          const float *bias, const double *lg, const uint64_t *bnd,
                                                          int nb, int E, int k, double bscale, int32_t *idx,
                                                          float *wout, int32_t *n_fixup) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const double B = bscale * bound_of_slots(bnd + t * nb, nb);  // bscale = topk_bound_scale(depth)
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
                            int64_t E, int k, int32_t *idx, float *w, int32_t *n_fixup, const RouterWs &rw,
                            bool want_logits) {
  constexpr int H = NC * 256;
  int depth, nb;
  if (T >= kBf16RouterMinT && !want_logits) {
    // candidates from the bf16 matrix cores, ranked on fp64 recomputed values
    const int nslots = (int)cdiv(E, 4);
    TMOE_LAUNCH(TMOE_KERNEL_ROUTER_LOGITS, router_split_kernel<NC>, dim3((unsigned)nslots), dim3(256), 0, st, Wr,
                bias, (int)E, rw.parts, rw.wmax, nslots, rw.wnorm, n_fixup);
    TMOE_LAUNCHED("router_split");
    const int64_t ntile = cdiv(T, 128) * cdiv(E, 128);
    if (ntile * kRgMaxSK > 0x7FFFFFFF) return fail(TMOE_E_UNSUPPORTED, "T too large");
    // input slices so that about 256 workgroups run (at least 4 K steps each)
    int SK = 1;
    while (SK < kRgMaxSK && ntile * SK < 256 && H / 32 / (2 * SK) >= 4) SK *= 2;
    const size_t lds = (size_t)kRgStages * kRgStage;
    const dim3 grid((unsigned)(ntile * SK));
    float *part = rw.part;
    int rc = SK == 1 ? allow_lds<router_gemm_kernel<1>>(lds)
                     : SK == 2 ? allow_lds<router_gemm_kernel<2>>(lds) : allow_lds<router_gemm_kernel<4>>(lds);
    if (rc) return rc;
    switch (SK) {
      case 1: TMOE_LAUNCH(TMOE_KERNEL_ROUTER_LOGITS, router_gemm_kernel<1>, grid, dim3(256), lds, st, X, T, rw.parts,
                          (int)E, H, (int)cdiv(E, 128), part); break;
      case 2: TMOE_LAUNCH(TMOE_KERNEL_ROUTER_LOGITS, router_gemm_kernel<2>, grid, dim3(256), lds, st, X, T, rw.parts,
                          (int)E, H, (int)cdiv(E, 128), part); break;
      default: TMOE_LAUNCH(TMOE_KERNEL_ROUTER_LOGITS, router_gemm_kernel<4>, grid, dim3(256), lds, st, X, T, rw.parts,
                           (int)E, H, (int)cdiv(E, 128), part); break;
    }
    TMOE_LAUNCHED("router_gemm");
    double gfac, babs;
    router_bf16_bound(H, SK, &gfac, &babs);
    TMOE_LAUNCH(TMOE_KERNEL_ROUTER_TOPK, (router_topk_refine_kernel<NPL, NC>), dim3((unsigned)cdiv(T, 4)), dim3(256), 0,
                st, T, X, Wr, bias, part, SK, rw.wmax, nslots, rw.wnorm, (int)E, k, gfac, babs, idx, w, n_fixup);
    TMOE_LAUNCHED("router_topk_refine");
    return TMOE_OK;
  }
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
              H, Wr, bias, rw.lg, rw.bnd, nb, (int)E, k, topk_bound_scale(depth), idx, w, n_fixup);
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
  const bool want = logits_out != nullptr;
  int rc = [&]() -> int {
    TMOE_ROUTER_DISPATCH(launch_router_nc, st, X, T, Wr, bias, E, k, idx, w, n_fixup, rw, want);
  }();
  if (rc || !logits_out) return rc;
  hipLaunchKernelGGL(copy_d2f_kernel, dim3((unsigned)cdiv(T * E, 256)), dim3(256), 0, st, rw.lg, T * E, logits_out);
  TMOE_LAUNCHED("logits_copy");
  return TMOE_OK;
}

}  // namespace tmoe
