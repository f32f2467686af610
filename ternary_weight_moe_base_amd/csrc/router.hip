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
#include "device_util.h"

namespace tmoe {

static constexpr int kTokChunkBytes = 65536;  // LDS bytes of bf16 activations per workgroup

size_t router_ws_bytes(int64_t T, int64_t E) {
  size_t o = 0;
  o = align_up(o + 64, 256);         // ctr
  o = align_up(o + T * 8, 256);      // bnd
  o = align_up(o + T * E * 8, 256);  // lg
  o = align_up(o + 4, 256);          // fix_count
  o = align_up(o + T * 4, 256);      // fix_list
  o = align_up(o + (2 * E + 1 + 3 * 16 * T) * 4, 256);  // grouping scratch of the router-only decode path
  return o;
}

RouterWs router_ws_carve(void *ws, int64_t T, int64_t E) {
  char *b = (char *)ws;
  RouterWs r;
  size_t o = 0;
  r.ctr = (uint32_t *)(b + o);
  o = align_up(o + 64, 256);
  r.bnd = (uint64_t *)(b + o);
  o = align_up(o + T * 8, 256);
  r.lg = (double *)(b + o);
  o = align_up(o + T * E * 8, 256);
  r.fix_count = (int32_t *)(b + o);
  o = align_up(o + 4, 256);
  r.fix_list = (int32_t *)(b + o);
  o = align_up(o + T * 4, 256);
  r.scratch = (int32_t *)(b + o);
  return r;
}

__device__ inline float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ inline double wave_sum_d(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ inline double gamma_d(int d) {
  const double u = 0x1p-53;
  return d * u / (1.0 - d * u);
}

// ------------------------------------------------------- double-double sums
// TwoSum (Knuth): s + e == a + b exactly, whatever the operand order.
__device__ inline void two_sum(double a, double b, double &s, double &e) {
  s = a + b;
  double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}
__device__ inline void dd_add(double &hi, double &lo, double v) {
  double s, e;
  two_sum(hi, v, s, e);
  e += lo;
  two_sum(s, e, hi, lo);
}
__device__ inline void dd_add_dd(double &hi, double &lo, double h2, double l2) {
  double s, e;
  two_sum(hi, h2, s, e);
  e += lo + l2;
  two_sum(s, e, hi, lo);
}

// ------------------------------------------------------------- wave top-k
// Values held NPL per lane (expert lane + 64 j). Order: larger value, then
// (for double-double values) larger low part, then lower expert index.
template <int NPL, bool DD>
struct TopM {
  double v[NPL], l[NPL];
  uint32_t taken = 0;

  __device__ void argmax(double &bv, double &bl, int &bi) {
    const int lane = threadIdx.x & 63;
    bv = -INFINITY;
    bl = 0.0;
    bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      if (taken & (1u << j)) continue;
      const int e = lane + 64 * j;  // grows with j: strict > keeps the lower index
      if (v[j] > bv || (DD && v[j] == bv && l[j] > bl) || bi == 0x7FFFFFFF) {
        bv = v[j];
        bl = DD ? l[j] : 0.0;
        bi = e;
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const double ov = __shfl_xor(bv, m, 64);
      const double ol = DD ? __shfl_xor(bl, m, 64) : 0.0;
      const int oi = __shfl_xor(bi, m, 64);
      const bool take = ov > bv || (ov == bv && ((DD && ol > bl) || ((!DD || ol == bl) && oi < bi)));
      if (take) {
        bv = ov;
        bl = ol;
        bi = oi;
      }
    }
    if ((bi & 63) == lane && bi != 0x7FFFFFFF) taken |= 1u << (bi >> 6);
  }

  // Ranks 0..m-1; lane r keeps rank r. Returns whether all adjacent gaps > gap.
  __device__ bool select(int m, double gap, double &myv, double &myl, int &myi, double &v0) {
    const int lane = threadIdx.x & 63;
    bool ok = true;
    double prev = 0.0;
    myv = -INFINITY;
    myl = 0.0;
    myi = 0;
    v0 = 0.0;
    for (int r = 0; r < m; ++r) {
      double bv, bl;
      int bi;
      argmax(bv, bl, bi);
      if (r == 0) v0 = bv;
      else ok = ok && (prev - bv > gap);
      prev = bv;
      if (r == lane) {
        myv = bv;
        myl = bl;
        myi = bi;
      }
    }
    return ok;
  }
};

// Softmax over the k selected (lane r holds rank r) -> idx / w of one token.
__device__ inline void write_topk(int k, double myv, double myl, int myi, double v0, int32_t *idx, float *w,
                                  int32_t *sidx) {
  const int lane = threadIdx.x & 63;
  const double p = lane < k ? exp((myv - v0) + myl) : 0.0;
  const double den = wave_sum_d(p);
  if (lane < k) {
    idx[lane] = myi;
    w[lane] = (float)(p / den);
    if (sidx) sidx[lane] = myi;
  }
}

// Certified top-k of one token by one wavefront from its fp64 logits.
template <int NPL>
__device__ inline bool topk_certified(const double *lg, int E, int k, double B, int32_t *idx, float *w,
                                      int32_t *sidx) {
  const int lane = threadIdx.x & 63;
  TopM<NPL, false> t;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + 64 * j;
    t.v[j] = e < E ? lg[e] : -INFINITY;
    t.l[j] = 0.0;
    if (e >= E) t.taken |= 1u << j;
  }
  double myv, myl, v0;
  int myi;
  if (!t.select(min(k + 1, E), 2.0 * B, myv, myl, myi, v0)) return false;
  write_topk(k, myv, 0.0, myi, v0, idx, w, sidx);
  return true;
}

// Double-double logits of one token by one wavefront (lane-strided partial
// sums, fixed butterfly: identical router rows give identical values), then
// top-k with ties to the lower index.
template <int NPL>
__device__ inline void topk_dd(const uint16_t *x, int H, const float *Wr, const float *bias, int E, int k,
                               int32_t *idx, float *w, int32_t *sidx) {
  const int lane = threadIdx.x & 63;
  TopM<NPL, true> t;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    t.v[j] = -INFINITY;
    t.l[j] = 0.0;
    if (lane + 64 * j >= E) t.taken |= 1u << j;
  }
  for (int e = 0; e < E; ++e) {
    const float *wr = Wr + (int64_t)e * H;
    double hi = 0.0, lo = 0.0;
    for (int i = lane; i < H; i += 64) dd_add(hi, lo, (double)bf16f(x[i]) * (double)wr[i]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      double oh = __shfl_xor(hi, m, 64), ol = __shfl_xor(lo, m, 64);
      dd_add_dd(hi, lo, oh, ol);
    }
    if (bias) dd_add(hi, lo, (double)bias[e]);
    if ((e & 63) == lane) {
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if (j == (e >> 6)) {
          t.v[j] = hi;
          t.l[j] = lo;
        }
    }
  }
  double myv, myl, v0;
  int myi;
  t.select(k, -1.0, myv, myl, myi, v0);
  write_topk(k, myv, myl, myi, v0, idx, w, sidx);
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
  for (int i = threadIdx.x; i < nt * vpr; i += blockDim.x) {
    int n = i / vpr, c = i % vpr;
    reinterpret_cast<uint4 *>(xs + (size_t)n * H)[c] = reinterpret_cast<const uint4 *>(X + (t0 + n) * H)[c];
  }
}

__device__ inline uint64_t dbits(double v) { return (uint64_t)__double_as_longlong(v); }
__device__ inline double bitsd(uint64_t b) { return __longlong_as_double((long long)b); }

// Workgroup = 4 wavefronts = 4 experts; grid.y walks token chunks.
template <int NC>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t *X, int64_t T, const float *Wr,
                                                            const float *bias, int64_t E, int tchunk, double *lg,
                                                            uint64_t *bnd, int32_t *fix_count) {
  extern __shared__ __align__(16) uint16_t xs[];
  __shared__ double lgs[4 * 128], abs_s[4 * 128];
  const int64_t e0 = (int64_t)blockIdx.x * 4;
  const int64_t t0 = (int64_t)blockIdx.y * tchunk;
  const int nt = (int)min<int64_t>(tchunk, T - t0);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *fix_count = 0;
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
    atomicMax((unsigned long long *)&bnd[t0 + n], (unsigned long long)dbits(a));
  }
}

// One wavefront per token; resets the token's bound slot for the next call.
template <int NPL>
__global__ __launch_bounds__(256) void router_topk_kernel(int64_t T, const double *lg, uint64_t *bnd, int E, int k,
                                                          int depth, int32_t *idx, float *wout, int32_t *fix_count,
                                                          int32_t *fix_list) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const double B = 1.01 * gamma_d(depth) * bitsd(bnd[t]);
  if (!topk_certified<NPL>(lg + t * E, E, k, B, idx + t * k, wout + t * k, nullptr) && lane == 0)
    fix_list[atomicAdd(fix_count, 1)] = (int32_t)t;
  if (lane == 0) bnd[t] = 0;
}

// Double-double recompute of the listed tokens (one wavefront per token).
template <int NPL>
__global__ __launch_bounds__(256) void router_fixup_kernel(const uint16_t *X, int H, const float *Wr,
                                                           const float *bias, int E, int k, const int32_t *fix_count,
                                                           const int32_t *fix_list, int32_t *idx, float *wout,
                                                           int32_t *n_fixup) {
  const int nfix = *fix_count;
  if (blockIdx.x == 0 && threadIdx.x == 0 && n_fixup) *n_fixup = nfix;
  const int wave = threadIdx.x >> 6;
  for (int i = blockIdx.x * 4 + wave; i < nfix; i += gridDim.x * 4) {
    const int64_t t = fix_list[i];
    topk_dd<NPL>(X + t * H, H, Wr, bias, E, k, idx + t * k, wout + t * k, nullptr);
  }
}

__global__ void copy_d2f_kernel(const double *a, int64_t n, float *b) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) b[i] = (float)a[i];
}

// ------------------------------------------- fused decode path (T <= 16)
// grid = ceil(E / 4) workgroups. All of them compute fp64 logits; thread 0 of
// each publishes them (one writer, then one device-scope release fence and a
// counter increment). The last workgroup to arrive (acquire fence) certifies
// the top-k of every token, groups the (token, slot) pairs by expert, writes
// the work tiles (one per hit expert, <= 16 pairs each), then resets the
// counter and bound slots for the next call.
struct DecodeOut {
  int32_t *idx;
  float *w;
  int32_t *n_fixup;
  int32_t *counts, *offsets, *sorted_token, *sorted_slot, *pos;
  int32_t *tiles, *ntiles;  // may be null (router-only use)
};

template <int NC, int NPL>
__global__ __launch_bounds__(256) void router_decode_kernel(const uint16_t *X, int T, const float *Wr,
                                                            const float *bias, int E, int k, RouterWs rw,
                                                            DecodeOut o) {
  constexpr int H = NC * 256;
  extern __shared__ __align__(16) char smem[];
  uint16_t *xs = reinterpret_cast<uint16_t *>(smem);  // [T][H]
  __shared__ double lgs[4 * 16], abs_s[4 * 16];
  __shared__ int last, nfix;
  __shared__ uint32_t bits[1024];
  __shared__ int32_t sidx[16 * 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t e0 = (int64_t)blockIdx.x * 4;
  stage_x(xs, X, 0, T, H);
  __syncthreads();
  logits_rows<NC>(xs, T, Wr, bias, e0 + wave, E, lgs, abs_s);
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int n = 0; n < T; ++n) {
      for (int q = 0; q < 4; ++q)
        if (e0 + q < E) rw.lg[(int64_t)n * E + e0 + q] = lgs[n * 4 + q];
      const double a = fmax(fmax(abs_s[n * 4], abs_s[n * 4 + 1]), fmax(abs_s[n * 4 + 2], abs_s[n * 4 + 3]));
      atomicMax((unsigned long long *)&rw.bnd[n], (unsigned long long)dbits(a));
    }
    __threadfence();
    last = atomicAdd(rw.ctr, 1u) == gridDim.x - 1;
    nfix = 0;
  }
  __syncthreads();
  if (!last) return;
  __threadfence();

  // certified top-k, one wavefront per token
  const int depth = 4 * NC + 8;
  for (int t = wave; t < T; t += 4) {
    const double B = 1.01 * gamma_d(depth) * bitsd(__hip_atomic_load(&rw.bnd[t], __ATOMIC_RELAXED,
                                                                     __HIP_MEMORY_SCOPE_AGENT));
    if (!topk_certified<NPL>(rw.lg + (int64_t)t * E, E, k, B, o.idx + t * k, o.w + t * k, sidx + t * k)) {
      if (lane == 0) atomicAdd(&nfix, 1);
      topk_dd<NPL>(xs + (size_t)t * H, H, Wr, bias, E, k, o.idx + t * k, o.w + t * k, sidx + t * k);
    }
  }
  for (int i = threadIdx.x; i < E; i += 256) bits[i] = 0;
  __syncthreads();
  if (threadIdx.x == 0 && o.n_fixup) *o.n_fixup = nfix;
  if ((int)threadIdx.x < T) rw.bnd[threadIdx.x] = 0;

  // grouping: bit t of bits[e] <=> token t chose e (T <= 16)
  if ((int)threadIdx.x < T)
    for (int j = 0; j < k; ++j) {
      const int ex = sidx[threadIdx.x * k + j];
      if (ex >= 0 && ex < E) atomicOr(&bits[ex], 1u << threadIdx.x);
    }
  __syncthreads();
  if (wave == 0) {
    // lane l owns experts l*NPL .. l*NPL + NPL - 1; wave prefix sums give the
    // pair offsets (counts) and the tile slots (hit experts)
    int c[NPL], run = 0, hit = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int ex = lane * NPL + j;
      c[j] = ex < E ? __popc(bits[ex]) : 0;
      run += c[j];
      hit += c[j] > 0;
    }
    int incl = run, incl_h = hit;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int a = __shfl_up(incl, m, 64), b = __shfl_up(incl_h, m, 64);
      if (lane >= m) {
        incl += a;
        incl_h += b;
      }
    }
    int off = incl - run, toff = incl_h - hit;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int ex = lane * NPL + j;
      if (ex < E) {
        o.counts[ex] = c[j];
        o.offsets[ex] = off;
        if (c[j] > 0) {
          if (o.tiles) reinterpret_cast<int4 *>(o.tiles)[toff] = make_int4(ex, off, c[j], 0);
          // scatter the pairs of this expert in token order
          uint32_t bm = bits[ex];
          int p = off;
          while (bm) {
            const int t = __ffs(bm) - 1;
            bm &= bm - 1;
            int j2 = 0;
            for (int jj = 0; jj < k; ++jj)
              if (sidx[t * k + jj] == ex) j2 = jj;
            o.sorted_token[p] = t;
            o.sorted_slot[p] = j2;
            o.pos[t * k + j2] = p;
            ++p;
          }
        }
        off += c[j];
        toff += c[j] > 0;
      }
    }
    if (lane == 63) {
      o.offsets[E] = incl;
      if (o.ntiles) *o.ntiles = incl_h;
    }
  }
  if (threadIdx.x == 0) *rw.ctr = 0u;  // ready for the next call
}

// ---------------------------------------------------------------- launchers
template <int NC, int NPL>
static int launch_router_nc(hipStream_t st, const uint16_t *X, int64_t T, const float *Wr, const float *bias,
                            int64_t E, int k, int32_t *idx, float *w, int32_t *n_fixup, const RouterWs &rw) {
  constexpr int H = NC * 256;
  int tchunk = kTokChunkBytes / (H * 2);
  if (tchunk > 128) tchunk = 128;
  if (tchunk > T) tchunk = (int)T;
  dim3 grid((unsigned)cdiv(E, 4), (unsigned)cdiv(T, tchunk));
  size_t lds = (size_t)tchunk * H * 2;
  TMOE_LAUNCH(TMOE_KERNEL_ROUTER_LOGITS, (router_logits_kernel<NC>), grid, dim3(256), lds, st, X, T, Wr, bias, E,
              tchunk, rw.lg, rw.bnd, rw.fix_count);
  TMOE_LAUNCHED("router_logits");
  const int depth = 4 * NC + 8;
  TMOE_LAUNCH(TMOE_KERNEL_ROUTER_TOPK, (router_topk_kernel<NPL>), dim3((unsigned)cdiv(T, 4)), dim3(256), 0, st, T,
              rw.lg, rw.bnd, (int)E, k, depth, idx, w, rw.fix_count, rw.fix_list);
  TMOE_LAUNCHED("router_topk");
  const unsigned fx = (unsigned)(T < 64 ? T : 64);
  TMOE_LAUNCH(TMOE_KERNEL_ROUTER_FIXUP, (router_fixup_kernel<NPL>), dim3(fx), dim3(256), 0, st, X, H, Wr, bias,
              (int)E, k, rw.fix_count, rw.fix_list, idx, w, n_fixup);
  TMOE_LAUNCHED("router_fixup");
  return TMOE_OK;
}

template <int NC, int NPL>
static int launch_decode_nc(hipStream_t st, const uint16_t *X, int64_t T, const float *Wr, const float *bias,
                            int64_t E, int k, const RouterWs &rw, const DecodeOut &o) {
  constexpr int H = NC * 256;
  const size_t lds = (size_t)T * H * 2;
  int rc = allow_lds<router_decode_kernel<NC, NPL>>(lds + 8192);
  if (rc) return rc;
  TMOE_LAUNCH(TMOE_KERNEL_ROUTER_LOGITS, (router_decode_kernel<NC, NPL>), dim3((unsigned)cdiv(E, 4)), dim3(256), lds,
              st, X, (int)T, Wr, bias, (int)E, k, rw, o);
  TMOE_LAUNCHED("router_decode");
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

int launch_router_decode(hipStream_t st, const uint16_t *X, int64_t T, int64_t H, const float *Wr, const float *bias,
                         int64_t E, int k, const RouterWs &rw, int32_t *idx, float *w, int32_t *n_fixup,
                         int32_t *counts, int32_t *offsets, int32_t *sorted_token, int32_t *sorted_slot, int32_t *pos,
                         int32_t *tiles, int32_t *ntiles) {
  if (T > kDecodeMaxT || T < 1) return fail(TMOE_E_UNSUPPORTED, "decode router needs 1 <= T <= 16");
  const DecodeOut o{idx, w, n_fixup, counts, offsets, sorted_token, sorted_slot, pos, tiles, ntiles};
  TMOE_ROUTER_DISPATCH(launch_decode_nc, st, X, T, Wr, bias, E, k, rw, o);
}

int launch_router(hipStream_t st, const uint16_t *X, int64_t T, int64_t H, const float *Wr, const float *bias,
                  int64_t E, int k, int32_t *idx, float *w, float *logits_out, int32_t *n_fixup, const RouterWs &rw) {
  if (T > 0x7FFFFFFF / 4) return fail(TMOE_E_UNSUPPORTED, "T too large");
  int rc;
  if (T <= kDecodeMaxT) {
    int32_t *sc = rw.scratch;
    rc = launch_router_decode(st, X, T, H, Wr, bias, E, k, rw, idx, w, n_fixup, sc, sc + E, sc + 2 * E + 1,
                              sc + 2 * E + 1 + 16 * T, sc + 2 * E + 1 + 32 * T, nullptr, nullptr);
  } else {
    rc = [&]() -> int { TMOE_ROUTER_DISPATCH(launch_router_nc, st, X, T, Wr, bias, E, k, idx, w, n_fixup, rw); }();
  }
  if (rc || !logits_out) return rc;
  hipLaunchKernelGGL(copy_d2f_kernel, dim3((unsigned)cdiv(T * E, 256)), dim3(256), 0, st, rw.lg, T * E, logits_out);
  TMOE_LAUNCHED("logits_copy");
  return TMOE_OK;
}

}  // namespace tmoe
