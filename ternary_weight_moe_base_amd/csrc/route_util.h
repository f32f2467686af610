// Device helpers of the certified top-k, shared by the router kernels and by
// the gate/up kernel's routing prologue: fp64 wave sums, the summation error
// bound gamma_d, double-double accumulation, wave top-k with certification.
//
// Error bound (Higham, "Accuracy and Stability of Numerical Algorithms",
// recursive summation with FMA): |fl(l_e) - l_e| <= gamma_d * (A_e + |b_e|),
// A_e = sum_i |x_i w_ei|, gamma_d = d u / (1 - d u), u = 2^-53, d = chain length
// + butterfly depth + 1 (bias) + margin. With A = max_e (A_e + |b_e|) one bound
// B = 1.01 gamma_d A serves the whole token: the top k+1 ranking is certified
// when each adjacent gap > 2B.
#pragma once
#include "device_util.h"

namespace tmoe {

__device__ inline uint64_t dbits(double v) { return (uint64_t)__double_as_longlong(v); }
__device__ inline double bitsd(uint64_t b) { return __longlong_as_double((long long)b); }

__device__ inline float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ inline double wave_sum_d(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Sum over the 64 lanes with DPP steps (lane pairs xor 1 and xor 2, half-row
// and row mirrors, then row broadcasts 15 and 31), read from lane 63 and
// returned to every lane: a fixed tree of depth 6.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_add_step(double v) {
  const uint64_t b = dbits(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROW_MASK, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROW_MASK, 0xF, false);
  return v + bitsd(((uint64_t)hi << 32) | lo);
}
__device__ inline double wave_sum_dpp(double v) {
  v = dpp_add_step<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_add_step<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_add_step<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_add_step<0x140, 0xF>(v);  // row_mirror
  v = dpp_add_step<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v = dpp_add_step<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  const uint64_t b = dbits(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
  return bitsd(((uint64_t)hi << 32) | lo);
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

// ------------------------------------------------ fast certified top-k
// Order-preserving 64-bit key of a double (larger value <=> larger key).
__device__ inline uint64_t okey(double v) {
  const uint64_t b = dbits(v);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
__device__ inline double from_okey(uint64_t k) {
  return bitsd((k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k);
}

__device__ inline double readlane_d(double v, int l) {
  const uint64_t b = dbits(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return bitsd(((uint64_t)hi << 32) | lo);
}

// One step of a wave max of 32-bit values with a DPP lane permutation (lanes
// outside ROW_MASK keep their value).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v) {
  // lanes outside ROW_MASK read 0, the identity of an unsigned maximum, which
  // lets the compiler fold the permutation into the max instruction itself
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
  return o > v ? o : v;
}

// Maximum over the 64 lanes, returned to every lane: swaps in pairs and quads,
// half-row and row mirrors (each lane then holds its row of 16), row
// broadcasts 15 and 31 (lane 63 then holds the wave), read from lane 63.
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_step<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_step<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_max_step<0x140, 0xF>(v);  // row_mirror
  v = dpp_max_step<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v = dpp_max_step<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ inline uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = (uint32_t)(v >> 32);
  const uint32_t mh = wave_max_u32(hi);
  const uint32_t ml = wave_max_u32(hi == mh ? (uint32_t)v : 0u);
  return ((uint64_t)mh << 32) | ml;
}

// Largest of a token's nb bound slots (fp64 bits, all >= 0), to every lane.
__device__ inline double bound_of_slots(const uint64_t *slots, int nb) {
  uint64_t m = 0;
  for (int j = threadIdx.x & 63; j < nb; j += 64) m = m > slots[j] ? m : slots[j];
  return __longlong_as_double((long long)wave_max_u64(m));
}

// One token's logits: lane l holds experts l*NPL + j (0 past E).
template <int NPL>
__device__ inline void topk_load(const double *lg, int E, double v[NPL]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane * NPL + j;
    v[j] = e < E ? lg[e] : 0.0;
  }
}

// Order keys of the logits held as by topk_load (0 past E).
template <int NPL>
__device__ inline void topk_keys(const double v[NPL], int E, uint64_t key[NPL]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < NPL; ++j) key[j] = lane * NPL + j < E ? okey(v[j]) : 0ull;
}

// Top m of the wavefront's 64 NPL order keys (lane l holds slots NPL l + j):
// the lane sorts its keys once (equal keys keep the lower j first), then each
// of the m rounds takes the wave maximum of the lane heads (high words, then
// low words among the lanes that share the highest high word; equal keys to
// the lowest lane) and the winner drops its head. Lane r < m receives the key
// of rank r and its slot. sj must hold 0..NPL-1 on entry.
template <int NPL>
__device__ inline void wave_top_u64(uint64_t key[NPL], int sj[NPL], int m, uint64_t &mykey, int &myslot) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int pass = 0; pass < NPL; ++pass)
#pragma unroll
    for (int j = pass & 1; j + 1 < NPL; j += 2)
      if (key[j] < key[j + 1]) {
        const uint64_t tk = key[j];
        key[j] = key[j + 1];
        key[j + 1] = tk;
        const int tj = sj[j];
        sj[j] = sj[j + 1];
        sj[j + 1] = tj;
      }
  mykey = 0ull;
  myslot = 0;
  for (int r = 0; r < m; ++r) {
    const uint32_t hi = (uint32_t)(key[0] >> 32), lo = (uint32_t)key[0];
    const uint32_t mh = wave_max_u32(hi);
    uint64_t cand = __ballot(hi == mh);
    uint32_t ml;
    if (__popcll(cand) == 1) {
      ml = (uint32_t)__builtin_amdgcn_readlane((int)lo, (int)__builtin_ctzll(cand));
    } else {
      ml = wave_max_u32(hi == mh ? lo : 0u);
      cand = __ballot(hi == mh && lo == ml);
    }
    const int wl = (int)__builtin_ctzll(cand);
    const int wj = __builtin_amdgcn_readlane(sj[0], wl);
    if (lane == wl) {
#pragma unroll
      for (int j = 0; j + 1 < NPL; ++j) {
        key[j] = key[j + 1];
        sj[j] = sj[j + 1];
      }
      key[NPL - 1] = 0ull;
    }
    if (lane == r) {
      mykey = ((uint64_t)mh << 32) | ml;
      myslot = wl * NPL + wj;
    }
  }
}

// Certified top-k of one token by one wavefront from its order keys. The lane's
// keys are sorted once; each of the k+1 rounds takes the wave maximum of the
// lanes' head keys (high words first; low words only among the lanes that
// share the highest high word), and among equal keys the lowest lane, then the
// lowest j, i.e. the lower expert index. Returns false,
// writing nothing, when an adjacent gap of the top k+1 is not above 2B.
// Otherwise lane r < k writes rank r: idx, and the softmax weight over the k
// (fp64, summed in rank order).
template <int NPL>
__device__ inline bool topk_select(uint64_t key[NPL], int E, int k, double B, int32_t *idx, float *w) {
  const int lane = threadIdx.x & 63;
  // sort the lane's keys in descending order (stable: equal keys keep the lower j first)
  int sj[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) sj[j] = j;
#pragma unroll
  for (int pass = 0; pass < NPL; ++pass)
#pragma unroll
    for (int j = pass & 1; j + 1 < NPL; j += 2)
      if (key[j] < key[j + 1]) {
        const uint64_t tk = key[j];
        key[j] = key[j + 1];
        key[j + 1] = tk;
        const int tj = sj[j];
        sj[j] = sj[j + 1];
        sj[j + 1] = tj;
      }
  const int m = min(k + 1, E);
  bool ok = true;
  double prev = 0.0, v0 = 0.0, myv = 0.0;
  int myi = 0;
  for (int r = 0; r < m; ++r) {
    // the lane's best is its head key; the winner lane drops its head
    const uint32_t hi = (uint32_t)(key[0] >> 32), lo = (uint32_t)key[0];
    const uint32_t mh = wave_max_u32(hi);
    uint64_t cand = __ballot(hi == mh);
    uint32_t ml;
    if (__popcll(cand) == 1) {
      ml = (uint32_t)__builtin_amdgcn_readlane((int)lo, (int)__builtin_ctzll(cand));
    } else {
      ml = wave_max_u32(hi == mh ? lo : 0u);
      cand = __ballot(hi == mh && lo == ml);
    }
    const int wl = (int)__builtin_ctzll(cand);
    const int wj = __builtin_amdgcn_readlane(sj[0], wl);
    if (lane == wl) {
#pragma unroll
      for (int j = 0; j + 1 < NPL; ++j) {
        key[j] = key[j + 1];
        sj[j] = sj[j + 1];
      }
      key[NPL - 1] = 0ull;
    }
    const double v = from_okey(((uint64_t)mh << 32) | ml);
    if (r == 0) v0 = v;
    else ok = ok && (prev - v > 2.0 * B);
    prev = v;
    if (lane == r) {
      myv = v;
      myi = wl * NPL + wj;
    }
  }
  if (!ok) return false;
  const double p = lane < k ? exp(myv - v0) : 0.0;
  double den = 0.0;
  for (int r = 0; r < k; ++r) den += readlane_d(p, r);
  if (lane < k) {
    idx[lane] = myi;
    w[lane] = (float)(p / den);
  }
  return true;
}

// Fast certified top-k on unique 32-bit keys. The key of expert e is its
// "bucket" (the logit rounded to fp32, order-preserving, with the low IB bits
// cleared: a non-decreasing function of the logit) above E - 1 - e in those
// bits, so keys are distinct, and a wave maximum needs one 32-bit pass per
// round and identifies the winner by equality. The buckets order the logits
// only coarsely; the result is that of the exact logits when
//  - no unselected expert shares the bucket of the last selected one (then
//    every unselected logit is strictly below every selected one), and
//  - the selected fp64 logits, read back from lg, decrease with every
//    adjacent gap above 2B (the same test as topk_select).
// Otherwise it returns false and writes nothing (about 0.1% of tokens with
// logits ~ N(0, 1); the caller then runs topk_select). When it returns true,
// idx and w are those topk_select writes: same ranks, same fp64 softmax.
// kLanes: the selected logits come from the lanes holding them (one latency
// chain fewer, for a single token) instead of a re-read of lg (cheaper when
// many wavefronts share the memory pipeline).
template <int NPL, bool kLanes = false>
__device__ inline bool topk_fast(const double v[NPL], const double *lg, int E, int k, double B, int32_t *idx,
                                 float *w) {
  constexpr int IB = NPL * 64 <= 256 ? 8 : (NPL * 64 <= 1024 ? 10 : 12);
  static_assert(NPL * 64 <= (1 << IB), "expert index must fit the low key bits");
  const int lane = threadIdx.x & 63;
  uint32_t key[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane * NPL + j;
    uint32_t u = __float_as_uint((float)v[j]);  // round to nearest: non-decreasing
    if (u == 0x80000000u) u = 0u;               // -0 and +0 share a bucket
    const uint32_t o = (u >> 31) ? ~u : (u | 0x80000000u);
    key[j] = e < E ? (((o >> IB) << IB) | (uint32_t)(E - 1 - e)) : 0u;
  }
  // descending within the lane
#pragma unroll
  for (int pass = 0; pass < NPL; ++pass)
#pragma unroll
    for (int j = pass & 1; j + 1 < NPL; j += 2)
      if (key[j] < key[j + 1]) {
        const uint32_t t = key[j];
        key[j] = key[j + 1];
        key[j + 1] = t;
      }
  const int m = min(k + 1, E);
  uint32_t mine = 0u;  // lane r: the key of rank r
  for (int r = 0; r < m; ++r) {
    const uint32_t mx = wave_max_u32(key[0]);  // > 0: fewer than E experts taken
    if (key[0] == mx) {                        // the one lane holding it
#pragma unroll
      for (int j = 0; j + 1 < NPL; ++j) key[j] = key[j + 1];
      key[NPL - 1] = 0u;
    }
    if (lane == r) mine = mx;
  }
  const uint32_t last = (uint32_t)__builtin_amdgcn_readlane((int)mine, m - 1);
  if (__ballot(key[0] >= ((last >> IB) << IB)) != 0ull) return false;  // bucket shared with an unselected expert
  const int myi = E - 1 - (int)(mine & ((1u << IB) - 1u));
  double myv;
  if constexpr (kLanes) {
    // slot myi = NPL * lane' + j' lives in lane' (every lane takes part in the
    // shuffles; lanes past m hold a valid index and discard the value)
    const int src = myi / NPL, sj = myi - src * NPL;
    double got = 0.0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const double t = __shfl(v[j], src, 64);
      got = j == sj ? t : got;
    }
    myv = lane < m ? got : 0.0;
  } else {
    myv = lane < m ? lg[myi] : 0.0;
  }
  const double nxt = __shfl_down(myv, 1, 64);
  if (__ballot(lane + 1 < m && !(myv - nxt > 2.0 * B)) != 0ull) return false;
  const double v0 = readlane_d(myv, 0);
  const double p = lane < k ? exp(myv - v0) : 0.0;
  double den = 0.0;
  for (int r = 0; r < k; ++r) den += readlane_d(p, r);
  if (lane < k) {
    idx[lane] = myi;
    w[lane] = (float)(p / den);
  }
  return true;
}

// Certified top-k of one token's logits lg[0..E) (also held as by topk_load)
// by one wavefront: the fast 32-bit path, then the 64-bit tournament. False:
// not certifiable in fp64.
template <int NPL, bool kLanes = false>
__device__ inline bool topk_certified_v(const double v[NPL], const double *lg, int E, int k, double B, int32_t *idx,
                                        float *w) {
  if (topk_fast<NPL, kLanes>(v, lg, E, k, B, idx, w)) return true;
  uint64_t key[NPL];
  topk_keys<NPL>(v, E, key);
  return topk_select<NPL>(key, E, k, B, idx, w);
}

template <int NPL>
__device__ inline bool topk_certified(const double *lg, int E, int k, double B, int32_t *idx, float *w) {
  double v[NPL];
  topk_load<NPL>(lg, E, v);
  return topk_certified_v<NPL>(v, lg, E, k, B, idx, w);
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


}  // namespace tmoe
