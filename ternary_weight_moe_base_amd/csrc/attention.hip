// Attention half of a layer: ternary q/k/v/o projections, rotary embedding on
// half of each head on sliding-window layers, none on global layers, and
// softmax attention over a key/value cache.
//
// The pages fix the pattern (ai.thesatyajit.com, "The architecture around the
// quantization"; jj-blog, architecture list): three layers with a 512-token
// sliding window and rotary embeddings on half the head dimension (partial
// rotary factor 0.5), then one global layer without positional encoding,
// repeated. The projection sizes follow from the parameter census
// (ai.thesatyajit.com, "The 5.31 GB claim reconciles"): 19.58B ternary
// parameters minus the experts leave 2 x 2048 x 2048 + 2 x 512 x 2048 per
// layer. Head count, head size, rotary base and pairing are not on the pages;
// the library takes them as parameters (the model shape uses 16 query heads,
// 4 key/value heads of 128, base 10000, pairs (i, i + rotary_dim / 2)).
//
// Data flow for T new tokens at positions pos0 .. pos0 + T - 1:
//   1. qkv = ternary linear of x (one pass over the stacked [q; k; v] rows)
//   2. rotary on q and k (sliding layers); k, v appended to the cache
//   3. per (token, key/value head, key split): the four query heads of the
//      group against the visible keys, online softmax, partial sums
//   4. the splits merged -> attention output, fp32
//   5. o = ternary linear of the fp32 attention output (three exact bf16
//      parts) and the residual x + o rounded to bf16
// Cache layout (fp32): K and V [kv_heads][capacity][head_dim] (one key's 512
// bytes contiguous, so a step's 64 keys arrive in one round of coalesced
// loads); position j lives in slot j mod capacity.
#include <cmath>

#include "common.h"
#include "device_util.h"

namespace tmoe {

namespace {

constexpr int kAttnHeadDim = 128;
constexpr int kAttnGroup = 4;    // query heads per key/value head = wavefronts per workgroup
constexpr int kAttnKeys = 64;    // keys per step of the online softmax
constexpr int kAttnMaxSplit = 128;
constexpr int kAttnKRow = kAttnHeadDim + 4;  // padded LDS row of a key: float4 reads of 16 lanes hit 64 banks
constexpr size_t kAttnLds = (size_t)kAttnKeys * (kAttnKRow + kAttnHeadDim) * 4;

__device__ inline float wave_max_f(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ inline float wave_sum_f(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Rotary inverse frequencies base^(-2i/rot), i < rot/2, computed on the host
// in fp64 and passed by value.
struct RopeFreq {
  double inv[kAttnHeadDim / 2];
};

// grid (T, nh + 2 nkv), block 64: one head of one token. Query and key heads
// turn their first `rot` dimensions (pairs (i, i + rot/2)) by p * inv_i: the
// angle is formed and reduced modulo 2 pi in fp64 (positions reach 2^17 and
// beyond), then its sine and cosine are taken in fp32. Queries go to qr
// [T][nh][hd], keys and values to cache slot p mod cap.
__global__ __launch_bounds__(64) void rope_append_kernel(const float *qkv, int nh, int nkv, int rot, RopeFreq fr,
                                                         int64_t pos0, float *qr, float *kc, float *vc, int64_t cap) {
  constexpr int hd = kAttnHeadDim;
  __shared__ float cs_s[kAttnHeadDim / 2][2];
  const int t = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int64_t p = pos0 + t;
  const int64_t slot = p % cap;
  const int half = rot / 2;
  const float *src = qkv + ((int64_t)t * (nh + 2 * nkv) + h) * hd;
  const float2 x = reinterpret_cast<const float2 *>(src)[lane];  // dimensions 2 lane, 2 lane + 1
  float2 y = x;
  if (h < nh + nkv && rot > 0) {
    if (lane < half) {
      const double twopi = 6.283185307179586476925286766559;
      const double ang = (double)p * fr.inv[lane];
      float sn, c;
      sincosf((float)(ang - twopi * rint(ang / twopi)), &sn, &c);
      cs_s[lane][0] = c;
      cs_s[lane][1] = sn;
    }
    __syncthreads();
    float v[2] = {x.x, x.y};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int dd = 2 * lane + e;
      if (dd < rot) {
        const int j = dd < half ? dd : dd - half;
        const float c = cs_s[j][0], sn = cs_s[j][1];
        const float x1 = src[j], x2 = src[j + half];
        v[e] = dd < half ? fmaf(x1, c, -x2 * sn) : fmaf(x2, c, x1 * sn);
      }
    }
    y = make_float2(v[0], v[1]);
  }
  float *dst;
  if (h < nh) dst = qr + ((int64_t)t * nh + h) * hd;
  else if (h < nh + nkv) dst = kc + ((int64_t)(h - nh) * cap + slot) * hd;
  else dst = vc + ((int64_t)(h - nh - nkv) * cap + slot) * hd;
  reinterpret_cast<float2 *>(dst)[lane] = y;
}

struct AttnArgs {
  const float *qr;  // [T][nh][hd] (fused one-token path: the raw q/k/v row instead)
  float *kc, *vc;  // written by the fused one-token path (its own position)
  float *part;  // [T][nh][nsplit][hd + 2]: acc[hd], running max, sum
  int64_t cap, pos0;
  int T, nh, nkv, window, nsplit;
  float scale;
  int rot;  // fused one-token path: rotated dimensions
};
// The one token's rotary cosines and sines (angles formed and reduced on the
// host in fp64), a kernel argument of its own so it is read in place.
struct RopeCS {
  float cs[kAttnHeadDim / 2][2];
};

// grid (T * nkv, nsplit), block 256: wavefront w is query head g*4 + w of
// key/value head g. The split's key range is walked 64 keys at a time: the
// step's keys and values are loaded into LDS by the whole workgroup in one
// round of coalesced 16-byte loads; lane j then scores key j for its head,
// the wavefront updates its running max and sum and rescales its
// accumulator, and each lane adds the probability-weighted values of its two
// dimensions.
//
// FUSED (one token): the rotary and the cache append happen here instead of
// in rope_append_kernel. Every workgroup rotates its four query heads from
// the raw q/k/v row; the one workgroup whose range holds the token's own
// position rotates the new key, stores key and value in the cache, and stages
// them from LDS in place of that (not yet written) cache slot. No other
// workgroup reads that slot: on sliding layers it held a position outside the
// window, on global layers it was empty.
template <bool FUSED>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a, RopeCS rcs) {
  constexpr int hd = kAttnHeadDim, HD4 = hd / 4;
  extern __shared__ __align__(16) float lds[];
  float(*ks)[kAttnKRow] = reinterpret_cast<float(*)[kAttnKRow]>(lds);
  float(*vs)[hd] = reinterpret_cast<float(*)[hd]>(lds + kAttnKeys * kAttnKRow);
  __shared__ float4 qs[kAttnGroup][HD4];
  __shared__ float ps[kAttnGroup][kAttnKeys];
  __shared__ float4 knew[HD4], vnew[HD4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x / a.nkv, g = blockIdx.x - t * a.nkv;
  const int h = g * kAttnGroup + wave;
  const int64_t p = a.pos0 + t;
  const int64_t lo = a.window > 0 && p - a.window + 1 > 0 ? p - a.window + 1 : 0;
  const int64_t nkeys = p - lo + 1;
  const int64_t per = (nkeys + a.nsplit - 1) / a.nsplit;
  const int64_t chunk = (per + kAttnKeys - 1) / kAttnKeys * kAttnKeys;
  const int64_t k0 = lo + (int64_t)blockIdx.y * chunk;
  const int64_t k1 = k0 + chunk < p + 1 ? k0 + chunk : p + 1;
  const float4 *kg = reinterpret_cast<const float4 *>(a.kc + (int64_t)g * a.cap * hd);
  const float4 *vg = reinterpret_cast<const float4 *>(a.vc + (int64_t)g * a.cap * hd);
  const bool own = FUSED && k0 <= p && p < k1;  // this workgroup's range holds the new position
  if (threadIdx.x < kAttnGroup * HD4) {
    float4 q = reinterpret_cast<const float4 *>(a.qr + ((int64_t)t * a.nh + g * kAttnGroup) * hd)[threadIdx.x];
    q.x *= a.scale;
    q.y *= a.scale;
    q.z *= a.scale;
    q.w *= a.scale;
    qs[threadIdx.x / HD4][threadIdx.x % HD4] = q;
  }
  if (own && threadIdx.x < 2 * HD4) {
    const float *row = a.qr + (int64_t)(a.nh + (threadIdx.x < HD4 ? 0 : a.nkv) + g) * hd;
    const float4 v = reinterpret_cast<const float4 *>(row)[threadIdx.x % HD4];
    if (threadIdx.x < HD4) knew[threadIdx.x] = v;
    else vnew[threadIdx.x - HD4] = v;
  }
  if (FUSED && a.rot > 0) {
    __syncthreads();
    // pairs (i, i + rot/2) of the four query heads and of the new key
    const int half = a.rot / 2;
    float *qf = reinterpret_cast<float *>(qs), *kf = reinterpret_cast<float *>(knew);
    for (int idx = threadIdx.x; idx < (kAttnGroup + 1) * half; idx += 256) {
      const int hh = idx / half, i = idx - hh * half;
      if (hh == kAttnGroup && !own) continue;
      float *x = hh < kAttnGroup ? qf + hh * hd : kf;
      const float c = rcs.cs[i][0], sn = rcs.cs[i][1];
      const float x1 = x[i], x2 = x[i + half];
      x[i] = fmaf(x1, c, -x2 * sn);
      x[i + half] = fmaf(x2, c, x1 * sn);
    }
  }
  if (own) {
    __syncthreads();
    const int64_t slot = p % a.cap;
    if (threadIdx.x < HD4)
      reinterpret_cast<float4 *>(a.kc)[((int64_t)g * a.cap + slot) * HD4 + threadIdx.x] = knew[threadIdx.x];
    else if (threadIdx.x < 2 * HD4)
      reinterpret_cast<float4 *>(a.vc)[((int64_t)g * a.cap + slot) * HD4 + threadIdx.x - HD4] =
          vnew[threadIdx.x - HD4];
  }
  float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int64_t base = k0; base < k1; base += kAttnKeys) {
    const int nv = (int)(k1 - base < kAttnKeys ? k1 - base : kAttnKeys);
    // the step's keys and values: 2 x 64 rows of 32 float4, eight per thread each
    float4 kv[8], vv[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int c = threadIdx.x + 256 * r, j = c / HD4, d4 = c - j * HD4;
      const int64_t slot = (base + (j < nv ? j : 0)) % a.cap;
      kv[r] = kg[slot * HD4 + d4];
      vv[r] = vg[slot * HD4 + d4];
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int c = threadIdx.x + 256 * r, j = c / HD4, d4 = c - j * HD4;
      // the new position comes from LDS (its cache slot is being written by this workgroup)
      float4 kx = kv[r], vx = vv[r];
      if (own && base + j == p) {  // value selects (a select of the two sources' addresses spills kv, vv)
        const float4 kn = knew[d4], vn = vnew[d4];
        kx = make_float4(kn.x, kn.y, kn.z, kn.w);
        vx = make_float4(vn.x, vn.y, vn.z, vn.w);
      }
      *reinterpret_cast<float4 *>(&ks[j][4 * d4]) = kx;
      *reinterpret_cast<float4 *>(&vs[j][4 * d4]) = vx;
    }
    __syncthreads();
    float dot = 0.f;
#pragma unroll
    for (int d4 = 0; d4 < HD4; ++d4) {
      const float4 k = *reinterpret_cast<const float4 *>(&ks[lane][4 * d4]);
      const float4 q = qs[wave][d4];
      dot = fmaf(q.x, k.x, dot);
      dot = fmaf(q.y, k.y, dot);
      dot = fmaf(q.z, k.z, dot);
      dot = fmaf(q.w, k.w, dot);
    }
    const bool valid = lane < nv;
    const float sc = valid ? dot : -INFINITY;
    const float mn = fmaxf(m, wave_max_f(sc));
    const float corr = __expf(m - mn);  // m = -inf on the first step: 0
    const float pj = valid ? __expf(sc - mn) : 0.f;
    l = l * corr + wave_sum_f(pj);
    acc0 *= corr;
    acc1 *= corr;
    m = mn;
    ps[wave][lane] = pj;  // read back by this wavefront only
    for (int j = 0; j < nv; ++j) {
      const float2 v = *reinterpret_cast<const float2 *>(&vs[j][2 * lane]);
      const float pw = ps[wave][j];
      acc0 = fmaf(pw, v.x, acc0);
      acc1 = fmaf(pw, v.y, acc1);
    }
    __syncthreads();  // before the next step overwrites the keys and values
  }
  float *o = a.part + (((int64_t)t * a.nh + h) * a.nsplit + blockIdx.y) * (hd + 2);
  reinterpret_cast<float2 *>(o)[lane] = make_float2(acc0, acc1);
  if (lane == 0) {
    o[hd] = m;  // -inf: the split saw no key
    o[hd + 1] = l;
  }
}

// grid T * nh, block 128 (one thread per dimension):
// out[d] = sum_s e^(m_s - M) acc_s[d] / sum_s e^(m_s - M) l_s over the splits
// that saw a key (M = max_s m_s); the split weights are formed once in LDS.
__global__ __launch_bounds__(128) void attn_merge_kernel(const float *part, int nsplit, float *out) {
  constexpr int hd = kAttnHeadDim;
  __shared__ float w_s[kAttnMaxSplit], red[2];
  const int64_t th = blockIdx.x;
  const float *pp = part + th * nsplit * (hd + 2);
  const int tid = threadIdx.x;
  const float ms = tid < nsplit ? pp[tid * (hd + 2) + hd] : -INFINITY;
  const float ls = tid < nsplit ? pp[tid * (hd + 2) + hd + 1] : 0.f;
  float M = wave_max_f(ms);
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(red[0], red[1]);
  const float w = ms == -INFINITY ? 0.f : __expf(ms - M);
  if (tid < nsplit) w_s[tid] = w;
  float den = wave_sum_f(w * ls);
  __syncthreads();  // red is reused
  if ((tid & 63) == 0) red[tid >> 6] = den;
  __syncthreads();
  den = red[0] + red[1];
  float num = 0.f;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) num = fmaf(w_s[s], pp[s * (hd + 2) + tid], num);
  out[th * hd + tid] = num / den;
}

}  // namespace

int attn_nsplit(int64_t T, int nkv) {
  int64_t n = (512 + T * nkv - 1) / (T * nkv);
  return (int)(n < 1 ? 1 : (n > kAttnMaxSplit ? kAttnMaxSplit : n));
}

size_t attn_ws_bytes(int64_t T, int nh, int nkv, int hd) {
  const int64_t width = (int64_t)(nh + 2 * nkv) * hd;
  size_t o = 0;
  o = align_up(o + T * width * 4, 256);                                   // qkv
  o = align_up(o + T * nh * hd * 4, 256);                                 // rotated queries
  o = align_up(o + (size_t)T * nh * attn_nsplit(T, nkv) * (hd + 2) * 4, 256);  // split partials
  o = align_up(o + T * nh * hd * 4, 256);                                 // attention output
  return o;
}

int launch_attention(hipStream_t st, const tmoe_attn_weights &sh, const uint16_t *X, int64_t T, int64_t pos0,
                     float *kc, float *vc, int64_t cap, float *O, uint16_t *X_out, void *ws) {
  const int nh = sh.n_heads, nkv = sh.n_kv_heads, hd = sh.head_dim;
  const int64_t width = (int64_t)(nh + 2 * nkv) * hd;
  char *b = (char *)ws;
  size_t off = 0;
  float *qkv = (float *)(b + off);
  off = align_up(off + T * width * 4, 256);
  float *qr = (float *)(b + off);
  off = align_up(off + T * nh * hd * 4, 256);
  float *part = (float *)(b + off);
  // splits of 64-key steps: at most what the workspace holds, and no more than the
  // longest visible range needs
  const int64_t reach = sh.window > 0 && sh.window < pos0 + T ? sh.window : pos0 + T;
  const int64_t need_split = (reach + kAttnKeys - 1) / kAttnKeys;
  const int ns_ws = attn_nsplit(T, nkv);
  const int nsplit = need_split < ns_ws ? (int)need_split : ns_ws;
  off = align_up(off + (size_t)T * nh * ns_ws * (hd + 2) * 4, 256);
  float *attn = (float *)(b + off);

  int rc = launch_linear(st, sh.qkv_p, sh.qkv_s, width, sh.hidden, X, sh.hidden, T, qkv, width, nullptr);
  if (rc) return rc;
  if (T > 0x7FFFFFFF / nkv) return fail(TMOE_E_UNSUPPORTED, "T too large");
  const int rot = sh.window > 0 ? sh.rotary_dim : 0;
  const bool fused = T == 1;
  AttnArgs a;
  a.rot = rot;
  RopeCS rcs{};
  if (fused) {
    // one token: its angles here in fp64 (reduced, then fp32); rotary and append in the attention kernel
    for (int i = 0; i < rot / 2; ++i) {
      const double ang = (double)pos0 * std::pow(sh.rope_base, -2.0 * i / rot);
      rcs.cs[i][0] = (float)std::cos(ang);
      rcs.cs[i][1] = (float)std::sin(ang);
    }
  } else {
    RopeFreq fr{};
    for (int i = 0; i < rot / 2; ++i) fr.inv[i] = std::pow(sh.rope_base, -2.0 * i / rot);
    hipLaunchKernelGGL(rope_append_kernel, dim3((unsigned)T, (unsigned)(nh + 2 * nkv)), dim3(64), 0, st, qkv, nh, nkv,
                       rot, fr, pos0, qr, kc, vc, cap);
    TMOE_LAUNCHED("rope_append");
  }
  a.qr = fused ? qkv : qr;
  a.kc = kc;
  a.vc = vc;
  a.part = part;
  a.cap = cap;
  a.pos0 = pos0;
  a.T = (int)T;
  a.nh = nh;
  a.nkv = nkv;
  a.window = sh.window;
  a.nsplit = nsplit;
  a.scale = 1.0f / sqrtf((float)hd);
  if (fused) {
    rc = allow_lds<attn_kernel<true>>(kAttnLds);
    if (rc) return rc;
    TMOE_LAUNCH(TMOE_KERNEL_ATTENTION, attn_kernel<true>, dim3((unsigned)nkv, (unsigned)nsplit), dim3(256), kAttnLds,
                st, a, rcs);
  } else {
    rc = allow_lds<attn_kernel<false>>(kAttnLds);
    if (rc) return rc;
    TMOE_LAUNCH(TMOE_KERNEL_ATTENTION, attn_kernel<false>, dim3((unsigned)(T * nkv), (unsigned)nsplit), dim3(256),
                kAttnLds, st, a, rcs);
  }
  TMOE_LAUNCHED("attention");
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)(T * nh)), dim3(hd), 0, st, part, nsplit, attn);
  TMOE_LAUNCHED("attention_merge");
  return launch_linear3(st, sh.o_p, sh.o_s, sh.hidden, (int64_t)nh * hd, attn, T, O, X_out ? X : nullptr, X_out);
}

}  // namespace tmoe
