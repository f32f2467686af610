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
// Kernels: lmh_logits (the stream: fp64 logits, per-workgroup maxima of the
// logits and of the bound sums), lmh_select (a threshold below the (k+1)-th
// logit from the per-workgroup maxima, and the ids at or above it),
// lmh_merge (exact ranking of those candidates, certification, fallbacks).
#include "route_util.h"

namespace tmoe {

constexpr int kLmhGrid = 1024;     // workgroups of lmh_logits: four per CU, all resident at once
constexpr int kLmhSelTokens = 1024;  // token ids scanned per workgroup of lmh_select
constexpr int kLmhSelCap = 64;     // candidates one lmh_select workgroup may keep
constexpr int kLmhCap = 2048;      // candidate ids ranked per token
constexpr int kLmhFallbackCap = 256;


struct LmhWs {
  int32_t *cnt;    // [T][nsel]: candidates found by each lmh_select workgroup
  double *lg;      // [T][V]
  float *am;       // [T][nblk]: per-workgroup max of sum |x w|
  uint64_t *bm;    // [T][nblk]: per-workgroup max order key of the logits
  uint64_t *ckey;  // [T][nsel][kLmhSelCap]
  int32_t *cidx;   // [T][nsel][kLmhSelCap]
};

// workgroups of lmh_logits: one batch of 4 / T rows per wavefront at least
static int64_t lmh_nblk(int64_t T, int64_t V) {
  const int64_t nb = cdiv(cdiv(V, 4 / T), 4);
  return nb < kLmhGrid ? nb : kLmhGrid;
}

static int64_t lmh_nsel(int64_t V) { return cdiv(V, kLmhSelTokens); }

static size_t lmh_ws_layout(void *ws, int64_t T, int64_t V, LmhWs *w) {
  const int64_t nblk = lmh_nblk(T, V), nsel = lmh_nsel(V);
  char *b = (char *)ws;
  size_t o = 0;
  if (w) w->cnt = (int32_t *)(b + o);
  o = align_up(o + (size_t)T * nsel * 4, 256);
  if (w) w->lg = (double *)(b + o);
  o = align_up(o + (size_t)T * V * 8, 256);
  if (w) w->am = (float *)(b + o);
  o = align_up(o + (size_t)T * nblk * 4, 256);
  if (w) w->bm = (uint64_t *)(b + o);
  o = align_up(o + (size_t)T * nblk * 8, 256);
  if (w) w->ckey = (uint64_t *)(b + o);
  o = align_up(o + (size_t)T * nsel * kLmhSelCap * 8, 256);
  if (w) w->cidx = (int32_t *)(b + o);
  o = align_up(o + (size_t)T * nsel * kLmhSelCap * 4, 256);
  return o;
}

size_t lmh_ws_bytes(int64_t T, int64_t V, int k) {
  (void)k;
  return lmh_ws_layout(nullptr, T, V, nullptr);
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

// Workgroup = 4 wavefronts; the batches of RB = 4 / T consecutive rows (RB x T
// = 4 values) are split evenly over all wavefronts of the grid, each taking a
// contiguous run; the grid is sized so that every workgroup is resident at
// once (no tail of late workgroups). Lane l holds the activations
// x[t][512 c + 8 l + j] in fp32 and reads, per row, the 16-byte pieces
// 512 c + 8 l .. +8 (each load instruction of the wavefront is one contiguous
// 1 KB run of the row).
template <int T, int NC>
__global__ __launch_bounds__(256) void lmh_logits_kernel(const uint16_t *X, const uint16_t *W, int64_t V, double *lg,
                                                         float *logits, float *am, uint64_t *bm) {
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
  const int64_t nbt = (V + RB - 1) / RB, nw = (int64_t)gridDim.x * 4, gw = (int64_t)blockIdx.x * 4 + wave;
  const int64_t b0 = gw * nbt / nw, b1 = (gw + 1) * nbt / nw;
  const int q = lane >> 4;         // the value this lane ends with
  const int qr = q / T, qt = q % T;
  float amax = 0.f;
  uint64_t kmax = 0ull;
  // rows past V repeat the last row; their sums are dropped
  auto load_batch = [&](int64_t r0, uint4 (&wv)[RB][NC]) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int64_t v = min(r0 + r, V - 1);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        // the table is read once per call: non-temporal loads keep it from displacing cached data
        const u32x4 t_ = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(W + v * H + c * 512 + lane * 8));
        wv[r][c] = make_uint4(t_[0], t_[1], t_[2], t_[3]);
      }
    }
  };
  for (int64_t bb = b0; bb < b1; ++bb) {
    const int64_t r0 = bb * RB;
    uint4 wv[RB][NC];
    load_batch(r0, wv);
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
      const uint64_t kk = okey(sum);
      kmax = kk > kmax ? kk : kmax;
    }
  }
  // per-workgroup maxima of the bound sums and of the logits, per token
  __shared__ float red[4][4];
  __shared__ uint64_t redk[4][4];
  if ((lane & 15) == 0) {
    red[wave][q] = amax;
    redk[wave][q] = kmax;
  }
  __syncthreads();
  if (threadIdx.x < T) {
    float mx = 0.f;
    uint64_t km = 0ull;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        if (qq % T == (int)threadIdx.x) {
          mx = fmaxf(mx, red[w][qq]);
          km = redk[w][qq] > km ? redk[w][qq] : km;
        }
    am[(int64_t)threadIdx.x * gridDim.x + blockIdx.x] = mx;
    bm[(int64_t)threadIdx.x * gridDim.x + blockIdx.x] = km;
  }
}

// ------------------------------------------------------------------ select
// Any m = k+1 of the per-workgroup maxima are m distinct logits, so the least
// of them lower-bounds the (k+1)-th logit. Lane l of wavefront 0 takes the
// maximum over the workgroups b with b mod 64 = l; tau, the m-th largest of
// these 64 lane maxima (m <= 64), is then at most the (k+1)-th logit: every
// id of the top k+1 has an order key >= tau (typically a few more than m ids
// do). Each workgroup computes the same tau (while its own logits are in
// flight), scans its 1024 ids and keeps those at or above it (count in cnt,
// up to kLmhSelCap of them in its own slots).
__global__ __launch_bounds__(256) void lmh_select_kernel(const double *lg, int64_t V, const uint64_t *bm, int nblk,
                                                         int m, int32_t *cnt, uint64_t *ckey, int32_t *cidx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.y, nsel = gridDim.x;
  __shared__ uint64_t s_max[256];
  __shared__ uint64_t s_tau;
  __shared__ int s_n;
  // this workgroup's logits first: in flight while tau is formed
  const int64_t v0 = (int64_t)blockIdx.x * kLmhSelTokens + threadIdx.x;
  double lv[kLmhSelTokens / 256];
#pragma unroll
  for (int j = 0; j < kLmhSelTokens / 256; ++j) {
    const int64_t v = v0 + 256 * j;
    lv[j] = v < V ? lg[(int64_t)t * V + v] : -INFINITY;
  }
  {
    uint64_t tk = 0ull;
    for (int b0 = threadIdx.x; b0 < nblk; b0 += 256 * 4) {
      uint64_t kb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) kb[j] = b0 + 256 * j < nblk ? bm[(int64_t)t * nblk + b0 + 256 * j] : 0ull;
#pragma unroll
      for (int j = 0; j < 4; ++j) tk = kb[j] > tk ? kb[j] : tk;
    }
    s_max[threadIdx.x] = tk;
  }
  if (threadIdx.x == 0) s_n = 0;
  __syncthreads();
  if (wave == 0) {
    uint64_t lk = 0ull;
#pragma unroll
    for (int w = 0; w < 4; ++w) lk = s_max[lane + 64 * w] > lk ? s_max[lane + 64 * w] : lk;
    uint64_t key[1] = {lk};
    int sj[1] = {0};
    uint64_t mykey;
    int myslot;
    wave_top_u64<1>(key, sj, m, mykey, myslot);
    const uint32_t th = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mykey >> 32), m - 1);
    const uint32_t tl = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mykey, m - 1);
    if (lane == 0) s_tau = ((uint64_t)th << 32) | tl;
  }
  __syncthreads();
  const uint64_t tau = s_tau;
  uint64_t *bk = ckey + ((int64_t)t * nsel + blockIdx.x) * kLmhSelCap;
  int32_t *bi = cidx + ((int64_t)t * nsel + blockIdx.x) * kLmhSelCap;
#pragma unroll
  for (int j = 0; j < kLmhSelTokens / 256; ++j) {
    const int64_t v = v0 + 256 * j;
    const uint64_t kv = okey(lv[j]);
    if (v < V && kv >= tau) {
      const int slot = atomicAdd(&s_n, 1);
      if (slot < kLmhSelCap) {
        bk[slot] = kv;
        bi[slot] = (int32_t)v;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) cnt[(int64_t)t * nsel + blockIdx.x] = s_n;
}

// ------------------------------------------------------------------- merge
struct LmhMergeArgs {
  const uint16_t *X, *W;
  int64_t V;
  int H;
  const double *lg;
  const float *am;
  int nblk, nsel;
  const int32_t *cnt;
  const uint64_t *ckey;
  const int32_t *cidx;
  int k;
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

// (key desc, id asc) order: whether (ka, ia) comes before (kb, ib)
__device__ inline bool lmh_before(uint64_t ka, int ia, uint64_t kb, int ib) { return ka > kb || (ka == kb && ia < ib); }

// One workgroup per token: the top m = k+1 of the candidates in (key desc,
// id asc) order by rank counting (or, when the candidate list overflowed, m
// passes of a workgroup-wide maximum over every id), certification, and the
// double-double fallback.
__global__ __launch_bounds__(256) void lmh_merge_kernel(LmhMergeArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x, m = a.k + 1;
  __shared__ uint64_t skey[kLmhCap + 8];
  __shared__ int32_t sid[kLmhCap + 8];
  __shared__ uint64_t topk_[64];
  __shared__ int32_t topi_[64];
  __shared__ float sred[256];
  __shared__ uint64_t rkey[256];
  __shared__ int32_t rid[256];
  __shared__ int32_t cand[kLmhFallbackCap];
  __shared__ double dhi[kLmhFallbackCap], dlo[kLmhFallbackCap];
  __shared__ int s_uncertain, s_cnt, s_over;
  __shared__ int s_off[256];
  __shared__ int s_boff[1024];
  __shared__ int s_tmp[256];
  __shared__ double s_lo;

  if (threadIdx.x == 0) {
    s_uncertain = 0;
    s_cnt = 0;
    s_over = 0;
  }
  __syncthreads();
  // candidate counts of the select workgroups (nsel <= 1024: up to 4 per thread)
  int c4[4], mine_n = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = threadIdx.x * 4 + j;
    c4[j] = b < a.nsel ? a.cnt[(int64_t)t * a.nsel + b] : 0;
  }
  float mx = 0.f;
  for (int i = threadIdx.x; i < a.nblk; i += 256) mx = fmaxf(mx, a.am[(int64_t)t * a.nblk + i]);
  sred[threadIdx.x] = mx;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (c4[j] > kLmhSelCap) s_over = 1;
    mine_n += min(c4[j], kLmhSelCap);
  }
  s_off[threadIdx.x] = mine_n;
  __syncthreads();
  const int n = block_exclusive_scan<256>(s_off, 256, s_tmp);
  for (int s = 128; s >= 1; s >>= 1) {
    if ((int)threadIdx.x < s) sred[threadIdx.x] = fmaxf(sred[threadIdx.x], sred[threadIdx.x + s]);
    __syncthreads();
  }
  const int depth = a.H / 64 + 8;  // per-lane chain of H / 64 terms, 6 butterfly levels, margin
  const double B = 1.02 * gamma_d(depth) * (double)sred[0];

  if (n <= kLmhCap && !s_over) {
    // per-select-workgroup offsets, then every kept slot copied by its own thread
    {
      int o = s_off[threadIdx.x];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int b = threadIdx.x * 4 + j;
        if (b < a.nsel) s_boff[b] = o;
        o += c4[j];
      }
    }
    __syncthreads();
    // candidate j: the last select workgroup b whose offset is <= j (binary search), slot j - off[b]
    for (int j = threadIdx.x; j < n; j += 256) {
      int lo = 0, hi = a.nsel - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_boff[mid] <= j) lo = mid;
        else hi = mid - 1;
      }
      const int64_t o = ((int64_t)t * a.nsel + lo) * kLmhSelCap + (j - s_boff[lo]);
      skey[j] = a.ckey[o];
      sid[j] = a.cidx[o];
    }
    // pad to a multiple of 8 with entries that precede no candidate
    const int n8 = (n + 7) & ~7;
    if ((int)threadIdx.x < n8 - n) {
      skey[n + threadIdx.x] = 0ull;
      sid[n + threadIdx.x] = 0x7FFFFFFF;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += 256) {
      const uint64_t ki = skey[i];
      const int ii = sid[i];
      int rank = 0;
      for (int j0 = 0; j0 < n8; j0 += 8) {
        uint64_t kj[8];
        int ij[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          kj[j] = skey[j0 + j];
          ij[j] = sid[j0 + j];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) rank += lmh_before(kj[j], ij[j], ki, ii);
      }
      if (rank < m) {
        topk_[rank] = ki;
        topi_[rank] = ii;
      }
    }
  } else {
    // too many ids at or above the threshold to keep:
    // m passes, each the (key desc, id asc) maximum of every id after the last taken
    uint64_t lk = ~0ull;
    int li = -1;
    for (int r = 0; r < m; ++r) {
      uint64_t bk = 0ull;
      int bi = 0x7FFFFFFF;
      for (int64_t v = threadIdx.x; v < a.V; v += 256) {
        const uint64_t kv = okey(a.lg[(int64_t)t * a.V + v]);
        if (lmh_before(lk, li, kv, (int)v) && lmh_before(kv, (int)v, bk, bi)) {
          bk = kv;
          bi = (int)v;
        }
      }
      rkey[threadIdx.x] = bk;
      rid[threadIdx.x] = bi;
      __syncthreads();
      for (int s = 128; s >= 1; s >>= 1) {
        if ((int)threadIdx.x < s && lmh_before(rkey[threadIdx.x + s], rid[threadIdx.x + s], rkey[threadIdx.x], rid[threadIdx.x])) {
          rkey[threadIdx.x] = rkey[threadIdx.x + s];
          rid[threadIdx.x] = rid[threadIdx.x + s];
        }
        __syncthreads();
      }
      lk = rkey[0];
      li = rid[0];
      if (threadIdx.x == 0) {
        topk_[r] = lk;
        topi_[r] = li;
      }
      __syncthreads();
    }
  }
  __syncthreads();

  if (wave == 0) {
    const uint64_t mykey = lane < m ? topk_[lane] : 0ull;
    const int myid = lane < m ? topi_[lane] : -1;
    // certification of the float64 ranking of the top k+1
    const double myv = from_okey(mykey);
    const double nv = __shfl_down(myv, 1, 64);
    const int nid = __shfl_down(myid, 1, 64);
    const bool pair = lane + 1 < m;
    const bool sep = pair && myv - nv > 2.0 * B;
    const bool eqv = pair && !sep && myv == nv;
    bool uncertain = __ballot(pair && !sep && !eqv) != 0ull;
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
  const int nf = min(s_cnt, kLmhFallbackCap);
  const bool overflow = s_cnt > kLmhFallbackCap;
  // candidates in token-id order (rank sort; ids are distinct)
  int my = 0, rank = 0;
  if ((int)threadIdx.x < nf) {
    my = cand[threadIdx.x];
    for (int i = 0; i < nf; ++i) rank += cand[i] < my;
  }
  __syncthreads();
  if ((int)threadIdx.x < nf) cand[rank] = my;
  __syncthreads();
  // double-double logits of the candidates (exact fp64 products, lane-strided sums, fixed butterfly)
  for (int i = wave; i < nf; i += 4) {
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
      tm.v[j] = c < nf ? dhi[c] : -INFINITY;
      tm.l[j] = c < nf ? dlo[c] : 0.0;
      if (c >= nf) tm.taken |= 1u << j;
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
              w.lg, logits, w.am, w.bm);
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
  LmhWs w;
  lmh_ws_layout(ws, T, V, &w);
  int rc;
  switch (T) {
    case 1: rc = launch_lmh_logits_h<1>(st, X, (int)H, W, V, logits, w); break;
    case 2: rc = launch_lmh_logits_h<2>(st, X, (int)H, W, V, logits, w); break;
    case 4: rc = launch_lmh_logits_h<4>(st, X, (int)H, W, V, logits, w); break;
    default: return fail(TMOE_E_UNSUPPORTED, "lm head: T must be 1, 2 or 4");
  }
  if (rc) return rc;
  const int nblk = (int)lmh_nblk(T, V), nsel = (int)lmh_nsel(V);
  TMOE_LAUNCH(TMOE_KERNEL_LMH_TOPK, lmh_select_kernel, dim3((unsigned)nsel, (unsigned)T), dim3(256), 0, st, w.lg, V,
              w.bm, nblk, k + 1, w.cnt, w.ckey, w.cidx);
  TMOE_LAUNCHED("lmh_select");
  LmhMergeArgs ma;
  ma.X = X;
  ma.W = W;
  ma.V = V;
  ma.H = (int)H;
  ma.lg = w.lg;
  ma.am = w.am;
  ma.nblk = nblk;
  ma.nsel = nsel;
  ma.cnt = w.cnt;
  ma.ckey = w.ckey;
  ma.cidx = w.cidx;
  ma.k = k;
  ma.idx = idx;
  ma.val = val;
  ma.n_fixup = n_fixup;
  TMOE_LAUNCH(TMOE_KERNEL_LMH_MERGE, lmh_merge_kernel, dim3((unsigned)T), dim3(256), 0, st, ma);
  TMOE_LAUNCHED("lmh_merge");
  return TMOE_OK;
}

}  // namespace tmoe
