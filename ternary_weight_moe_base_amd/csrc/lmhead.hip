// LM head: logits of the untied bf16 output embedding over the vocabulary and
// the certified top-k next tokens.
//
// ai.thesatyajit.com, "The 5.31 GB claim reconciles, and the leftover is the
// vocabulary": the model's input and output embedding tables (151,936 tokens
// x 2048) are untied and stay un-quantized; at two bytes an entry the output
// table alone is 622 MB, five times the packed expert bytes one token reads,
// so the head is a pure HBM stream. Its logits decide the next token, so the
// selection is made exact like the router's:
//  - logits l[t][v] = sum_i x[t][i] W[v][i]; every bf16 x bf16 product is
//    exact in fp32 and is added in fp64 (a fixed tree per logit, the same for
//    every row, so identical rows give identical values);
//  - with the per-token bound B = 1.02 gamma_d max_v sum_i |x_i W_vi| on the
//    fp64 error (Higham, recursive summation; gamma_d = d u / (1 - d u)), the
//    float64 ranking of the top k+1 is certified when each adjacent gap
//    exceeds 2B, or the two values are equal and their rows are identical;
//  - otherwise every token whose float64 logit reaches the (k+1)-th minus 2B
//    is recomputed in double-double and ranked by that value (ties to the
//    lower token id).
// Kernels: lmh_logits (the stream: fp64 logits and per-workgroup bound
// maxima), lmh_chunk_topk (top-(k+1) of each 512-token chunk, float64 order),
// lmh_merge (merge of the chunk lists, certification, rare fallback).
#include "route_util.h"

namespace tmoe {

constexpr int kLmhIter = 8;        // 4-value batches per wavefront in lmh_logits
constexpr int kLmhNpl = 8;         // values per lane in a chunk (512 tokens per chunk)
constexpr int kLmhChunk = 64 * kLmhNpl;
constexpr int kLmhMergeNpl = 8;    // chunk lists per lane in the merge (<= 512 chunks)
constexpr int kLmhFallbackCap = 256;

__host__ __device__ inline int lmh_rows_per_wg(int T) { return 4 * kLmhIter * (4 / T); }

struct LmhWs {
  double *lg;      // [T][V]
  float *am;       // [T][nblk]: per-workgroup max of sum |x w|
  uint64_t *ckey;  // [T][nchunks][m]
  int32_t *cidx;   // [T][nchunks][m]
};

static int64_t lmh_nblk(int64_t T, int64_t V) { return cdiv(V, lmh_rows_per_wg((int)T)); }

size_t lmh_ws_bytes(int64_t T, int64_t V, int k) {
  const int64_t nblk = lmh_nblk(T, V), nch = cdiv(V, kLmhChunk), m = k + 1;
  size_t o = 0;
  o = align_up(o + (size_t)T * V * 8, 256);
  o = align_up(o + (size_t)T * nblk * 4, 256);
  o = align_up(o + (size_t)T * nch * m * 8, 256);
  o = align_up(o + (size_t)T * nch * m * 4, 256);
  return o;
}

static LmhWs lmh_ws_carve(void *ws, int64_t T, int64_t V, int k) {
  const int64_t nblk = lmh_nblk(T, V), nch = cdiv(V, kLmhChunk), m = k + 1;
  char *b = (char *)ws;
  LmhWs w;
  size_t o = 0;
  w.lg = (double *)(b + o);
  o = align_up(o + (size_t)T * V * 8, 256);
  w.am = (float *)(b + o);
  o = align_up(o + (size_t)T * nblk * 4, 256);
  w.ckey = (uint64_t *)(b + o);
  o = align_up(o + (size_t)T * nch * m * 8, 256);
  w.cidx = (int32_t *)(b + o);
  return w;
}

// ------------------------------------------------------------------ logits
// Sum over the wavefront of four values per lane, transposed: lane l ends with
// the full sum of value q = 2 (l >> 5 & 1) + (l >> 4 & 1). Every value is
// reduced by the same pairing tree (lane l with l ^ 32, then 16, 8, 4, 2, 1),
// and each pairwise sum is commutative, so equal inputs give equal sums
// whichever slot q they occupy.
template <typename V>
__device__ inline V wave_sum4_transposed(V a0, V a1, V a2, V a3) {
  const int lane = threadIdx.x & 63;
  const bool h5 = lane & 32, h4 = lane & 16;
  V k0 = h5 ? a2 : a0, k1 = h5 ? a3 : a1;  // kept
  V s0 = h5 ? a0 : a2, s1 = h5 ? a1 : a3;  // sent
  k0 += __shfl_xor(s0, 32, 64);
  k1 += __shfl_xor(s1, 32, 64);
  V k = h4 ? k1 : k0, s = h4 ? k0 : k1;
  k += __shfl_xor(s, 16, 64);
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) k += __shfl_xor(k, m, 64);
  return k;
}

// Workgroup = 4 wavefronts; a wavefront takes kLmhIter batches of RB = 4 / T
// consecutive rows (RB x T = 4 values). Lane l holds the activations
// x[t][512 c + 8 l + j] in fp32 and reads, per row, the 16-byte pieces
// 512 c + 8 l .. +8 (each load instruction of the wavefront is one contiguous
// 1 KB run of the row).
template <int T, int NC>
__global__ __launch_bounds__(256) void lmh_logits_kernel(const uint16_t *X, const uint16_t *W, int64_t V, double *lg,
                                                         float *logits, float *am) {
  constexpr int H = 512 * NC, RB = 4 / T;
  static_assert(RB * T == 4, "four (row, token) values per batch");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float xs[T][NC][8];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 v = *reinterpret_cast<const uint4 *>(X + (int64_t)t * H + c * 512 + lane * 8);
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xs[t][c][2 * i] = __uint_as_float(d[i] << 16);
        xs[t][c][2 * i + 1] = __uint_as_float(d[i] & 0xFFFF0000u);
      }
    }
  const int64_t rbase = (int64_t)blockIdx.x * lmh_rows_per_wg(T) + (int64_t)wave * kLmhIter * RB;
  const int q = lane >> 4;         // the value this lane ends with
  const int qr = q / T, qt = q % T;
  float amax = 0.f;
  for (int it = 0; it < kLmhIter; ++it) {
    const int64_t r0 = rbase + (int64_t)it * RB;
    if (r0 >= V) break;
    uint4 wv[RB][NC];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int64_t v = min(r0 + r, V - 1);  // rows past V repeat the last row; their sums are dropped
#pragma unroll
      for (int c = 0; c < NC; ++c) wv[r][c] = *reinterpret_cast<const uint4 *>(W + v * H + c * 512 + lane * 8);
    }
    double acc[4];
    float aab[4];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int t = 0; t < T; ++t) {
        double s = 0.0;
        float sa = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const uint32_t d[4] = {wv[r][c].x, wv[r][c].y, wv[r][c].z, wv[r][c].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float w0 = __uint_as_float(d[i] << 16), w1 = __uint_as_float(d[i] & 0xFFFF0000u);
            s += (double)(w0 * xs[t][c][2 * i]);  // bf16 x bf16: exact in fp32
            s += (double)(w1 * xs[t][c][2 * i + 1]);
            sa = fmaf(fabsf(w0), fabsf(xs[t][c][2 * i]), sa);
            sa = fmaf(fabsf(w1), fabsf(xs[t][c][2 * i + 1]), sa);
          }
        }
        acc[r * T + t] = s;
        aab[r * T + t] = sa;
      }
    const double sum = wave_sum4_transposed<double>(acc[0], acc[1], acc[2], acc[3]);
    const float asum = wave_sum4_transposed<float>(aab[0], aab[1], aab[2], aab[3]);
    const int64_t v = r0 + qr;
    if ((lane & 15) == 0 && v < V) {
      lg[(int64_t)qt * V + v] = sum;
      if (logits) logits[(int64_t)qt * V + v] = (float)sum;
      amax = fmaxf(amax, asum);
    }
  }
  // per-workgroup maxima of the bound sums, per token
  __shared__ float red[4][4];
  if ((lane & 15) == 0) red[wave][q] = amax;
  __syncthreads();
  if (threadIdx.x < T) {
    float mx = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        if (qq % T == (int)threadIdx.x) mx = fmaxf(mx, red[w][qq]);
    am[(int64_t)threadIdx.x * gridDim.x + blockIdx.x] = mx;
  }
}

// -------------------------------------------------------------- chunk top
// Top m (float64 order, equal values to the lower token id) of each chunk of
// 64 NPL tokens, one wavefront per chunk; lane l holds tokens
// chunk base + NPL l + j. Ranks past the chunk's real tokens get key 0, id -1.
template <int NPL>
__global__ __launch_bounds__(256) void lmh_chunk_topk_kernel(const double *lg, int64_t V, int nchunks, int m,
                                                             uint64_t *ckey, int32_t *cidx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.y, c = blockIdx.x * 4 + wave;
  if (c >= nchunks) return;
  const int64_t v0 = (int64_t)c * 64 * NPL + lane * NPL;
  uint64_t key[NPL];
  int sj[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    key[j] = v0 + j < V ? okey(lg[(int64_t)t * V + v0 + j]) : 0ull;
    sj[j] = j;
  }
  uint64_t mykey;
  int myslot;
  wave_top_u64<NPL>(key, sj, m, mykey, myslot);
  if (lane < m) {
    const int64_t o = ((int64_t)t * nchunks + c) * m + lane;
    const int64_t v = (int64_t)c * 64 * NPL + myslot;
    ckey[o] = mykey;
    cidx[o] = (mykey != 0ull && v < V) ? (int32_t)v : -1;
  }
}

// ------------------------------------------------------------------- merge
struct LmhMergeArgs {
  const uint16_t *X, *W;
  int64_t V;
  int H;
  const double *lg;
  const float *am;
  int nblk;
  const uint64_t *ckey;
  const int32_t *cidx;
  int nchunks, k;
  int32_t *idx;
  float *val;
  int32_t *n_fixup;
};

// Whether rows a and b of W are bitwise identical (one wavefront).
__device__ inline bool rows_equal(const uint16_t *W, int H, int64_t a, int64_t b) {
  const int lane = threadIdx.x & 63;
  bool eq = true;
  for (int i = lane; i < H / 8; i += 64) {
    const uint4 x = reinterpret_cast<const uint4 *>(W + a * H)[i], y = reinterpret_cast<const uint4 *>(W + b * H)[i];
    eq = eq && x.x == y.x && x.y == y.y && x.z == y.z && x.w == y.w;
  }
  return __ballot(!eq) == 0ull;
}

// One workgroup per token: merge of the chunk lists (wavefront 0, lane l owns
// chunks NPL l + j), certification, and the double-double fallback.
template <int NPL>
__global__ __launch_bounds__(256) void lmh_merge_kernel(LmhMergeArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x, m = a.k + 1, nc = a.nchunks;
  uint64_t *skey = reinterpret_cast<uint64_t *>(smem);
  int32_t *sidx = reinterpret_cast<int32_t *>(smem + (size_t)nc * m * 8);
  __shared__ float sred[256];
  __shared__ int32_t cand[kLmhFallbackCap];
  __shared__ double dhi[kLmhFallbackCap], dlo[kLmhFallbackCap];
  __shared__ int s_uncertain, s_cnt;
  __shared__ double s_lo;

  for (int i = threadIdx.x; i < nc * m; i += 256) {
    skey[i] = a.ckey[(int64_t)t * nc * m + i];
    sidx[i] = a.cidx[(int64_t)t * nc * m + i];
  }
  float mx = 0.f;
  for (int i = threadIdx.x; i < a.nblk; i += 256) mx = fmaxf(mx, a.am[(int64_t)t * a.nblk + i]);
  sred[threadIdx.x] = mx;
  if (threadIdx.x == 0) {
    s_uncertain = 0;
    s_cnt = 0;
  }
  __syncthreads();
  for (int s = 128; s >= 1; s >>= 1) {
    if ((int)threadIdx.x < s) sred[threadIdx.x] = fmaxf(sred[threadIdx.x], sred[threadIdx.x + s]);
    __syncthreads();
  }
  const int depth = a.H / 64 + 8;  // per-lane chain of H / 64 terms, 6 butterfly levels, margin
  const double B = 1.02 * gamma_d(depth) * (double)sred[0];

  uint64_t mykey = 0ull;
  int myid = -1;
  if (wave == 0) {
    int ptr[NPL];
    uint64_t head[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int c = lane * NPL + j;
      ptr[j] = 0;
      head[j] = c < nc ? skey[c * m] : 0ull;
    }
    for (int r = 0; r < m; ++r) {
      // the lane's best head (lower j on equal keys: lower token ids)
      uint64_t best = head[0];
      int bj = 0;
#pragma unroll
      for (int j = 1; j < NPL; ++j)
        if (head[j] > best) {
          best = head[j];
          bj = j;
        }
      const uint32_t hi = (uint32_t)(best >> 32), lo = (uint32_t)best;
      const uint32_t mh = wave_max_u32(hi);
      uint64_t cand_l = __ballot(hi == mh);
      uint32_t ml;
      if (__popcll(cand_l) == 1) {
        ml = (uint32_t)__builtin_amdgcn_readlane((int)lo, (int)__builtin_ctzll(cand_l));
      } else {
        ml = wave_max_u32(hi == mh ? lo : 0u);
        cand_l = __ballot(hi == mh && lo == ml);
      }
      const int wl = (int)__builtin_ctzll(cand_l);
      int vid = -1;
      if (lane == wl) {
        int pj = 0;
#pragma unroll
        for (int j = 0; j < NPL; ++j)
          if (j == bj) pj = ptr[j];
        const int c = lane * NPL + bj;
        vid = sidx[c * m + pj];
#pragma unroll
        for (int j = 0; j < NPL; ++j)
          if (j == bj) {
            ptr[j] = pj + 1;
            head[j] = pj + 1 < m ? skey[c * m + pj + 1] : 0ull;
          }
      }
      vid = __builtin_amdgcn_readlane(vid, wl);
      if (lane == r) {
        mykey = ((uint64_t)mh << 32) | ml;
        myid = vid;
      }
    }
    // certification of the float64 ranking of the top k+1
    const double myv = from_okey(mykey);
    const double nv = __shfl_down(myv, 1, 64);
    const int nid = __shfl_down(myid, 1, 64);
    const bool pair = lane + 1 < m;
    const bool sep = pair && myv - nv > 2.0 * B;
    const bool eqv = pair && !sep && myv == nv;
    bool uncertain = __ballot(pair && !sep && !eqv) != 0ull || __ballot(myid < 0 && lane < m) != 0ull;
    uint64_t ties = __ballot(eqv);
    while (!uncertain && ties) {
      const int l = (int)__builtin_ctzll(ties);
      ties &= ties - 1;
      const int ra = __builtin_amdgcn_readlane(myid, l), rb = __builtin_amdgcn_readlane(nid, l);
      if (!rows_equal(a.W, a.H, ra, rb)) uncertain = true;
    }
    if (lane == 0) {
      s_uncertain = uncertain ? 1 : 0;
      s_lo = readlane_d(myv, m - 1) - 2.0 * B;
    }
    if (!uncertain && lane < a.k) {
      a.idx[(int64_t)t * a.k + lane] = myid;
      a.val[(int64_t)t * a.k + lane] = (float)myv;
    }
  }
  __syncthreads();
  if (!s_uncertain) return;

  // fallback: every token whose float64 logit reaches the (k+1)-th minus 2B
  const double lo = s_lo;
  for (int64_t v0 = threadIdx.x; v0 < a.V; v0 += 256 * 8) {
    double lv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t v = v0 + 256 * j;
      lv[j] = v < a.V ? a.lg[(int64_t)t * a.V + v] : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (lv[j] >= lo) {
        const int p = atomicAdd(&s_cnt, 1);
        if (p < kLmhFallbackCap) cand[p] = (int32_t)(v0 + 256 * j);
      }
  }
  __syncthreads();
  const int n = min(s_cnt, kLmhFallbackCap);
  const bool overflow = s_cnt > kLmhFallbackCap;
  // candidates in token-id order (rank sort; ids are distinct)
  int my = 0, rank = 0;
  if ((int)threadIdx.x < n) {
    my = cand[threadIdx.x];
    for (int i = 0; i < n; ++i) rank += cand[i] < my;
  }
  __syncthreads();
  if ((int)threadIdx.x < n) cand[rank] = my;
  __syncthreads();
  // double-double logits of the candidates (exact fp64 products, lane-strided sums, fixed butterfly)
  for (int i = wave; i < n; i += 4) {
    const int64_t row = cand[i];
    double hi = 0.0, lo2 = 0.0;
    for (int kk = lane; kk < a.H; kk += 64)
      dd_add(hi, lo2, (double)bf16f(a.X[(int64_t)t * a.H + kk]) * (double)bf16f(a.W[row * a.H + kk]));
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1) {
      const double oh = __shfl_xor(hi, msk, 64), ol = __shfl_xor(lo2, msk, 64);
      dd_add_dd(hi, lo2, oh, ol);
    }
    if (lane == 0) {
      dhi[i] = hi;
      dlo[i] = lo2;
    }
  }
  __syncthreads();
  if (wave == 0) {
    TopM<kLmhFallbackCap / 64, true> tm;
#pragma unroll
    for (int j = 0; j < kLmhFallbackCap / 64; ++j) {
      const int c = lane + 64 * j;
      tm.v[j] = c < n ? dhi[c] : -INFINITY;
      tm.l[j] = c < n ? dlo[c] : 0.0;
      if (c >= n) tm.taken |= 1u << j;
    }
    double sv, sl, v0;
    int si;
    tm.select(a.k, -1.0, sv, sl, si, v0);
    if (lane < a.k) {
      a.idx[(int64_t)t * a.k + lane] = cand[si];
      a.val[(int64_t)t * a.k + lane] = (float)(sv + sl);
    }
    if (lane == 0 && a.n_fixup) atomicAdd(a.n_fixup, overflow ? 65536 : 1);
  }
}

// ------------------------------------------------------------------ launch
template <int T, int NC>
static int launch_lmh_logits(hipStream_t st, const uint16_t *X, const uint16_t *W, int64_t V, float *logits,
                             const LmhWs &w) {
  const int64_t nblk = lmh_nblk(T, V);
  if (nblk > 0x7FFFFFFF) return fail(TMOE_E_UNSUPPORTED, "vocabulary too large");
  TMOE_LAUNCH(TMOE_KERNEL_LMH_LOGITS, (lmh_logits_kernel<T, NC>), dim3((unsigned)nblk), dim3(256), 0, st, X, W, V,
              w.lg, logits, w.am);
  TMOE_LAUNCHED("lmh_logits");
  return TMOE_OK;
}

template <int T>
static int launch_lmh_logits_h(hipStream_t st, const uint16_t *X, int H, const uint16_t *W, int64_t V, float *logits,
                               const LmhWs &w) {
  switch (H) {
    case 512: return launch_lmh_logits<T, 1>(st, X, W, V, logits, w);
    case 1024: return launch_lmh_logits<T, 2>(st, X, W, V, logits, w);
    case 2048: return launch_lmh_logits<T, 4>(st, X, W, V, logits, w);
    case 4096: return launch_lmh_logits<T, 8>(st, X, W, V, logits, w);
    default: return fail(TMOE_E_UNSUPPORTED, "lm head: hidden must be 512, 1024, 2048 or 4096");
  }
}

int launch_lm_head(hipStream_t st, const uint16_t *X, int64_t T, int64_t H, const uint16_t *W, int64_t V, int k,
                   int32_t *idx, float *val, float *logits, int32_t *n_fixup, void *ws) {
  const LmhWs w = lmh_ws_carve(ws, T, V, k);
  int rc;
  switch (T) {
    case 1: rc = launch_lmh_logits_h<1>(st, X, (int)H, W, V, logits, w); break;
    case 2: rc = launch_lmh_logits_h<2>(st, X, (int)H, W, V, logits, w); break;
    case 4: rc = launch_lmh_logits_h<4>(st, X, (int)H, W, V, logits, w); break;
    default: return fail(TMOE_E_UNSUPPORTED, "lm head: T must be 1, 2 or 4");
  }
  if (rc) return rc;
  const int nch = (int)cdiv(V, kLmhChunk), m = k + 1;
  TMOE_LAUNCH(TMOE_KERNEL_LMH_TOPK, lmh_chunk_topk_kernel<kLmhNpl>, dim3((unsigned)cdiv(nch, 4), (unsigned)T),
              dim3(256), 0, st, w.lg, V, nch, m, w.ckey, w.cidx);
  TMOE_LAUNCHED("lmh_chunk_topk");
  LmhMergeArgs ma;
  ma.X = X;
  ma.W = W;
  ma.V = V;
  ma.H = (int)H;
  ma.lg = w.lg;
  ma.am = w.am;
  ma.nblk = (int)lmh_nblk(T, V);
  ma.ckey = w.ckey;
  ma.cidx = w.cidx;
  ma.nchunks = nch;
  ma.k = k;
  ma.idx = idx;
  ma.val = val;
  ma.n_fixup = n_fixup;
  const size_t lds = (size_t)nch * m * 12;
  rc = allow_lds<lmh_merge_kernel<kLmhMergeNpl>>(lds + 8192);  // the kernel's static LDS comes on top
  if (rc) return rc;
  TMOE_LAUNCH(TMOE_KERNEL_LMH_MERGE, lmh_merge_kernel<kLmhMergeNpl>, dim3((unsigned)T), dim3(256), lds, st, ma);
  TMOE_LAUNCHED("lmh_merge");
  return TMOE_OK;
}

int lmh_max_chunks() { return 64 * kLmhMergeNpl; }
int lmh_chunk_tokens() { return kLmhChunk; }

}  // namespace tmoe
