// Ternary GEMV/GEMM kernels on MFMA: the ternary linear, the fused
// gate/up + SiLU/clamp expert half, the down projection, and the combine.
//
// Arithmetic (codeinsider.com.br, "Pesos ternarios": a ternary weight adds,
// subtracts or skips its input; ai.thesatyajit.com, "The shipped code does no
// quantization": out = linear(act(clamp(x Wg^T, max=7)) * clamp(x Wu^T, -7, 7), Wd)):
//  - A trit t enters the matrix core as the 16-bit value 2t, whose bit pattern
//    ((d - 1) mod 4) << 14 (d = t + 1 the base-3 digit) is the same in bf16
//    and fp16: 0xC000 = -2, 0 = 0, 0x4000 = +2. Products with bf16 or fp16
//    operands are exact; MFMA accumulates in fp32; the result is halved.
//  - Digits are decoded two bytes at a time in packed fp16: a byte pair b0, b1
//    becomes the fp16 pair (1024 + b0, 1024 + b1); one packed FMA computes
//    1024 + floor(R / 3) (rounding to the integer grid of [1024, 2048) is the
//    floor), another 1027 + R + floor(R / 3), whose two low bits are
//    (d - 1) mod 4 because d = R - 3 floor(R / 3) == R + floor(R / 3) (mod 4).
//  - gate/up take the bf16 activations directly. The down projection's input h
//    is fp32: it is scaled by a power of two and split into two fp16 parts
//    hi + lo (22 significant bits), each multiplied exactly.
#include "device_util.h"

namespace tmoe {

// ---------------------------------------------------------- trit decoding
__device__ __forceinline__ uint32_t fma16x2(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2, a),
                                                                __builtin_bit_cast(f16x2, b),
                                                                __builtin_bit_cast(f16x2, c)));
}
__device__ __forceinline__ uint32_t shl14x2(uint32_t w) {
  u16x2 v = __builtin_bit_cast(u16x2, w);
  v = v << (unsigned short)14;
  return __builtin_bit_cast(uint32_t, v);
}
// ((v + 3) << 14) per 16-bit half
__device__ __forceinline__ uint32_t top_digit_x2(uint32_t w) {
  u16x2 v = __builtin_bit_cast(u16x2, w);
  v = v * (unsigned short)0x4000 + (unsigned short)0xC000;
  return __builtin_bit_cast(uint32_t, v);
}

// fp16 constants (two copies per dword)
#define K_THIRD 0x35553555u  // 0.333251953125
#define K_C1 0x61556155u     // 682.5
#define K_43 0x3D553D55u     // 1.3330078125
#define K_C2 0xDD49DD49u     // -338.25

// Five pair-words (digits q = 0..4 of both bytes) from v = fp16 (1024 + b0, 1024 + b1).
__device__ __forceinline__ void digits5(uint32_t v, uint32_t *pw) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    pw[q] = shl14x2(fma16x2(v, K_43, K_C2));
    v = fma16x2(v, K_THIRD, K_C1);
  }
  pw[4] = top_digit_x2(v);
}
// bytes 0,1 (lo) or 2,3 (hi) of d as fp16 (1024 + b) pairs
__device__ __forceinline__ uint32_t pair_lo(uint32_t d) { return __builtin_amdgcn_perm(0x64646464u, d, 0x04010400u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t d) { return __builtin_amdgcn_perm(0x64646464u, d, 0x04030402u); }

// 8 bytes of one step -> 20 pair-words; MFMA m of the step uses pw[4m .. 4m+3]
__device__ __forceinline__ void unpack8(uint2 d, uint32_t pw[20]) {
  digits5(pair_lo(d.x), pw);
  digits5(pair_hi(d.x), pw + 5);
  digits5(pair_lo(d.y), pw + 10);
  digits5(pair_hi(d.y), pw + 15);
}

// Tail of RT bytes (2, 4, 6): dw holds bytes 0-3 (RT >= 4), sh bytes 4-5 or 0-1.
template <int RT>
__device__ __forceinline__ void unpack_tail(uint32_t dw, uint32_t sh, uint32_t pw[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) pw[i] = 0;
  if constexpr (RT >= 4) {
    digits5(pair_lo(dw), pw);
    digits5(pair_hi(dw), pw + 5);
    if constexpr (RT == 6) digits5(pair_lo(sh), pw + 10);
  } else if constexpr (RT == 2) {
    digits5(pair_lo(sh), pw);
  }
}

template <int RT>
__device__ __forceinline__ void load_tail(const uint8_t *tile, int F, int lane, uint32_t &dw, uint32_t &sh) {
  dw = 0;
  sh = 0;
  if constexpr (RT >= 4) dw = *reinterpret_cast<const uint32_t *>(tile + (int64_t)F * 512 + lane * 4);
  if constexpr (RT == 2 || RT == 6)
    sh = *reinterpret_cast<const uint16_t *>(tile + (int64_t)F * 512 + (RT >= 4 ? 256 : 0) + lane * 2);
}

constexpr int tail_mfmas(int RT) { return RT == 0 ? 0 : (5 * (RT / 2) + 3) / 4; }

__device__ __forceinline__ f32x4 mfma_bf16(const uint32_t *a, u32x4 b, f32x4 c) {
  u32x4 av = {a[0], a[1], a[2], a[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(const uint32_t *a, u32x4 b, f32x4 c) {
  u32x4 av = {a[0], a[1], a[2], a[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}

__device__ __forceinline__ u32x4 lds16(const char *p) { return *reinterpret_cast<const u32x4 *>(p); }

// LDS row stride (bytes) of a staged operand row with `slots` 16-bit values:
// slots/2 dwords is a multiple of 16; +4 dwords makes the 16 token rows start
// in 16 different 4-bank groups of the 64 LDS banks.
__host__ __device__ inline int lds_row_bytes(int slots) { return slots * 2 + 16; }

// ----------------------------------------------------- operand permutation
// xp[t][slot] = X[t][slot_to_k(slot)] (0 for pad slots): the activations in
// the order the MFMA B operand reads them.
__global__ void permute_x_kernel(const uint16_t *X, int64_t ldx, int64_t T, Geom g, uint16_t *xp) {
  const int64_t t = blockIdx.x;
  const int slot = blockIdx.y * 256 + threadIdx.x;
  if (t >= T || slot >= g.slots) return;
  int64_t k = slot_to_k(g, slot);
  xp[t * g.slots + slot] = k >= 0 ? X[t * ldx + k] : (uint16_t)0;
}

// One workgroup per grouped pair p: h row -> power-of-two scale 2^e with
// max|h| 2^-e in [2^14, 2^15), then fp16 hi = rn(h'), lo = rn(h' - hi) in
// down-operand order.
__global__ __launch_bounds__(256) void permute_h_kernel(const float *Hn, int I, const int32_t *offsets, int E,
                                                         Geom g, uint16_t *hp_hi, uint16_t *hp_lo, int32_t *hexp,
                                                         int64_t pairs) {
  __shared__ float red[4];
  const int64_t p = blockIdx.x;
  if (p >= pairs || p >= offsets[E]) return;
  const float *h = Hn + p * I;
  float m = 0.f;
  for (int i = threadIdx.x; i < I; i += 256) m = fmaxf(m, fabsf(h[i]));
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int e = 0;
  if (m > 0.f && m < INFINITY) e = ilogbf(m) - 14;
  if (threadIdx.x == 0) hexp[p] = e;
  for (int slot = threadIdx.x; slot < g.slots; slot += 256) {
    int64_t k = slot_to_k(g, slot);
    float v = k >= 0 ? ldexpf(h[k], -e) : 0.f;
    _Float16 hi = (_Float16)v;
    _Float16 lo = (_Float16)(v - (float)hi);
    hp_hi[p * g.slots + slot] = __builtin_bit_cast(uint16_t, hi);
    hp_lo[p * g.slots + slot] = __builtin_bit_cast(uint16_t, lo);
  }
}

// ---------------------------------------------------------------- tiles
// Work tiles of up to 16 grouped pairs of one expert, in expert order.
__global__ __launch_bounds__(256) void make_tiles_kernel(const int32_t *offsets, int E, int32_t *tiles,
                                                          int32_t *ntiles) {
  __shared__ int nt[1024];
  __shared__ int tmp[256];
  for (int e = threadIdx.x; e < E; e += 256) nt[e] = (offsets[e + 1] - offsets[e] + 15) / 16;
  __syncthreads();
  int total = block_exclusive_scan<256>(nt, E, tmp);
  for (int e = threadIdx.x; e < E; e += 256) {
    int c = offsets[e + 1] - offsets[e], base = nt[e];
    for (int i = 0; 16 * i < c; ++i) {
      int4 tv = make_int4(e, offsets[e] + 16 * i, min(16, c - 16 * i), 0);
      reinterpret_cast<int4 *>(tiles)[base + i] = tv;
    }
  }
  if (threadIdx.x == 0) *ntiles = total;
}

// ----------------------------------------------------------- gate / up
struct GateUpArgs {
  const uint8_t *gate_p, *up_p;
  int64_t stride_gu;
  const float *gate_s, *up_s;
  const uint16_t *xp;  // [T][slots]
  const int32_t *tiles, *ntiles, *sorted_token;
  float *h;  // [pairs][I]
  int I, slots;
  float clamp;
};

__device__ __forceinline__ float silu(float z) { return z / (1.f + expf(-z)); }

// Workgroup = 4 wavefronts. KS wavefronts split the K steps of one 16-row tile
// (partial sums reduced in LDS in fixed order); 4/KS row tiles per workgroup.
// blockIdx.x = work tile (expert, <= 16 pairs), blockIdx.y = row-tile group.
template <int F, int RT, int KS>
__global__ __launch_bounds__(256) void gateup_kernel(GateUpArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int tile = blockIdx.x;
  if (tile >= *a.ntiles) return;
  const int4 td = reinterpret_cast<const int4 *>(a.tiles)[tile];
  const int e = td.x, start = td.y, cnt = td.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int RTB = 4 / KS;
  constexpr int M = 5 * F + tail_mfmas(RT);
  constexpr int SMAX = (F + KS - 1) / KS;
  const int rt = blockIdx.y * RTB + wave / KS;
  const int kp = wave % KS;
  const int rs = lds_row_bytes(a.slots);
  char *xs = smem;  // [17][rs]; row 16 = zeros

  // weights first: all loads of this wavefront are in flight while x is staged
  const int64_t tbytes = 64 * (int64_t)(8 * F + RT);
  const uint8_t *gt = a.gate_p + (int64_t)e * a.stride_gu + (int64_t)rt * tbytes;
  const uint8_t *ut = a.up_p + (int64_t)e * a.stride_gu + (int64_t)rt * tbytes;
  const int s0 = kp * F / KS, s1 = (kp + 1) * F / KS;
  uint2 gd[SMAX], ud[SMAX];
#pragma unroll
  for (int i = 0; i < SMAX; ++i) {
    if (s0 + i < s1) {
      gd[i] = *reinterpret_cast<const uint2 *>(gt + (int64_t)(s0 + i) * 512 + lane * 8);
      ud[i] = *reinterpret_cast<const uint2 *>(ut + (int64_t)(s0 + i) * 512 + lane * 8);
    }
  }
  uint32_t gdw = 0, gsh = 0, udw = 0, ush = 0;
  const bool tail_here = RT > 0 && kp == KS - 1;
  if (tail_here) {
    load_tail<RT>(gt, F, lane, gdw, gsh);
    load_tail<RT>(ut, F, lane, udw, ush);
  }

  const int vpr = a.slots / 8;
  for (int i = threadIdx.x; i < cnt * vpr; i += 256) {
    int n = i / vpr, c = i - n * vpr;
    int64_t tok = a.sorted_token[start + n];
    *reinterpret_cast<uint4 *>(xs + n * rs + c * 16) = reinterpret_cast<const uint4 *>(a.xp + tok * a.slots)[c];
  }
  for (int c = threadIdx.x; c < vpr; c += 256) *reinterpret_cast<uint4 *>(xs + 16 * rs + c * 16) = make_uint4(0, 0, 0, 0);
  __syncthreads();

  const int n = lane & 15, g = lane >> 4;
  const char *bp = xs + (n < cnt ? n : 16) * rs + g * M * 16;
  f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < SMAX; ++i) {
    const int s = s0 + i;
    if (s < s1) {
      uint32_t pg[20], pu[20];
      unpack8(gd[i], pg);
      unpack8(ud[i], pu);
#pragma unroll
      for (int m = 0; m < 5; ++m) {
        u32x4 bx = lds16(bp + (5 * s + m) * 16);
        accg = mfma_bf16(pg + 4 * m, bx, accg);
        accu = mfma_bf16(pu + 4 * m, bx, accu);
      }
    }
  }
  if constexpr (RT > 0) {
    if (tail_here) {
      uint32_t pg[16], pu[16];
      unpack_tail<RT>(gdw, gsh, pg);
      unpack_tail<RT>(udw, ush, pu);
#pragma unroll
      for (int m = 0; m < tail_mfmas(RT); ++m) {
        u32x4 bx = lds16(bp + (5 * F + m) * 16);
        accg = mfma_bf16(pg + 4 * m, bx, accg);
        accu = mfma_bf16(pu + 4 * m, bx, accu);
      }
    }
  }
  if constexpr (KS > 1) {
    float *red = reinterpret_cast<float *>(smem + 17 * rs);  // [4 waves][64 lanes][8]
    float *mine = red + (wave * 64 + lane) * 8;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      mine[v] = accg[v];
      mine[4 + v] = accu[v];
    }
    __syncthreads();
    if (kp != 0) return;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      accg[v] = 0.f;
      accu[v] = 0.f;
    }
    for (int q = 0; q < KS; ++q) {
      const float *o = red + ((wave + q) * 64 + lane) * 8;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        accg[v] += o[v];
        accu[v] += o[4 + v];
      }
    }
  }
  if (n >= cnt) return;
  const int row0 = rt * 16 + 4 * g;
  const float4 sg = *reinterpret_cast<const float4 *>(a.gate_s + (int64_t)e * a.I + row0);
  const float4 su = *reinterpret_cast<const float4 *>(a.up_s + (int64_t)e * a.I + row0);
  const float sgv[4] = {sg.x, sg.y, sg.z, sg.w}, suv[4] = {su.x, su.y, su.z, su.w};
  float hv[4];
  const float c = a.clamp;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float gg = (accg[v] * 0.5f) * sgv[v];
    float uu = (accu[v] * 0.5f) * suv[v];
    hv[v] = silu(fminf(gg, c)) * fminf(fmaxf(uu, -c), c);
  }
  *reinterpret_cast<float4 *>(a.h + (int64_t)(start + n) * a.I + row0) = make_float4(hv[0], hv[1], hv[2], hv[3]);
}

// ----------------------------------------------------------------- down
struct DownArgs {
  const uint8_t *down_p;
  int64_t stride_d;
  const float *down_s;
  const uint16_t *hp_hi, *hp_lo;  // [pairs][slots]
  const int32_t *hexp;
  const int32_t *tiles, *ntiles;
  float *O;  // [pairs][H]
  int H, slots;
};

// Workgroup = 4 wavefronts x one 16-row tile each (64 output rows).
template <int F, int RT>
__global__ __launch_bounds__(256) void down_kernel(DownArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int tile = blockIdx.x;
  if (tile >= *a.ntiles) return;
  const int4 td = reinterpret_cast<const int4 *>(a.tiles)[tile];
  const int e = td.x, start = td.y, cnt = td.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int M = 5 * F + tail_mfmas(RT);
  const int rt = blockIdx.y * 4 + wave;
  const int rs = lds_row_bytes(a.slots);
  char *xh = smem;            // [17][rs]
  char *xl = smem + 17 * rs;  // [17][rs]

  const int64_t tbytes = 64 * (int64_t)(8 * F + RT);
  const uint8_t *dt = a.down_p + (int64_t)e * a.stride_d + (int64_t)rt * tbytes;
  uint2 dd[F];
#pragma unroll
  for (int s = 0; s < F; ++s) dd[s] = *reinterpret_cast<const uint2 *>(dt + (int64_t)s * 512 + lane * 8);
  uint32_t ddw = 0, dsh = 0;
  if constexpr (RT > 0) load_tail<RT>(dt, F, lane, ddw, dsh);

  const int vpr = a.slots / 8;
  for (int i = threadIdx.x; i < cnt * vpr; i += 256) {
    int n = i / vpr, c = i - n * vpr;
    int64_t p = start + n;
    *reinterpret_cast<uint4 *>(xh + n * rs + c * 16) = reinterpret_cast<const uint4 *>(a.hp_hi + p * a.slots)[c];
    *reinterpret_cast<uint4 *>(xl + n * rs + c * 16) = reinterpret_cast<const uint4 *>(a.hp_lo + p * a.slots)[c];
  }
  for (int c = threadIdx.x; c < vpr; c += 256) {
    *reinterpret_cast<uint4 *>(xh + 16 * rs + c * 16) = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4 *>(xl + 16 * rs + c * 16) = make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  const int n = lane & 15, g = lane >> 4;
  const int boff = (n < cnt ? n : 16) * rs + g * M * 16;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < F; ++s) {
    uint32_t pw[20];
    unpack8(dd[s], pw);
#pragma unroll
    for (int m = 0; m < 5; ++m) {
      acc = mfma_f16(pw + 4 * m, lds16(xh + boff + (5 * s + m) * 16), acc);
      acc = mfma_f16(pw + 4 * m, lds16(xl + boff + (5 * s + m) * 16), acc);
    }
  }
  if constexpr (RT > 0) {
    uint32_t pw[16];
    unpack_tail<RT>(ddw, dsh, pw);
#pragma unroll
    for (int m = 0; m < tail_mfmas(RT); ++m) {
      acc = mfma_f16(pw + 4 * m, lds16(xh + boff + (5 * F + m) * 16), acc);
      acc = mfma_f16(pw + 4 * m, lds16(xl + boff + (5 * F + m) * 16), acc);
    }
  }
  if (n >= cnt) return;
  const int64_t p = start + n;
  const int ex = a.hexp[p] - 1;  // the trits entered as 2t
  const int row0 = rt * 16 + 4 * g;
  const float4 sd = *reinterpret_cast<const float4 *>(a.down_s + (int64_t)e * a.H + row0);
  float4 o;
  o.x = ldexpf(acc[0], ex) * sd.x;
  o.y = ldexpf(acc[1], ex) * sd.y;
  o.z = ldexpf(acc[2], ex) * sd.z;
  o.w = ldexpf(acc[3], ex) * sd.w;
  *reinterpret_cast<float4 *>(a.O + p * a.H + row0) = o;
}

// ---------------------------------------------------------- ternary linear
struct LinearArgs {
  const uint8_t *pt;
  const float *s;
  const uint16_t *xp;  // [T][slots]
  float *Y;
  int64_t T, N, ldy;
  int slots;
  Geom g;  // used by the generic (F < 0) instance
};

// blockIdx.x = 16-token tile, blockIdx.y = group of 4/KS row tiles. F < 0:
// generic K (runtime steps, one step in flight).
template <int F, int RT, int KS>
__global__ __launch_bounds__(256) void linear_kernel(LinearArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int RTB = 4 / KS;
  const int64_t t0 = (int64_t)blockIdx.x * 16;
  const int cnt = (int)min<int64_t>(16, a.T - t0);
  const int nrt = (int)((a.N + 15) / 16);
  const int rt = blockIdx.y * RTB + wave / KS;
  const int kp = wave % KS;
  const bool active = rt < nrt;
  const int rs = lds_row_bytes(a.slots);
  const int Fr = F >= 0 ? F : a.g.F;
  const int Rr = F >= 0 ? RT : a.g.r;
  const int M = 5 * Fr + (Rr == 0 ? 0 : (5 * (Rr / 2) + 3) / 4);
  const int64_t tbytes = 64 * (int64_t)(8 * Fr + Rr);
  const uint8_t *wt = a.pt + (int64_t)(active ? rt : 0) * tbytes;
  char *xs = smem;

  const int vpr = a.slots / 8;
  for (int i = threadIdx.x; i < cnt * vpr; i += 256) {
    int n = i / vpr, c = i - n * vpr;
    *reinterpret_cast<uint4 *>(xs + n * rs + c * 16) = reinterpret_cast<const uint4 *>(a.xp + (t0 + n) * a.slots)[c];
  }
  for (int c = threadIdx.x; c < vpr; c += 256) *reinterpret_cast<uint4 *>(xs + 16 * rs + c * 16) = make_uint4(0, 0, 0, 0);
  __syncthreads();

  const int n = lane & 15, g = lane >> 4;
  const char *bp = xs + (n < cnt ? n : 16) * rs + g * M * 16;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int s0 = kp * Fr / KS, s1 = (kp + 1) * Fr / KS;
  const bool tail_here = Rr > 0 && kp == KS - 1;
  if (active) {
    if constexpr (F >= 0) {
      constexpr int SMAX = (F + KS - 1) / KS;
      uint2 d[SMAX > 0 ? SMAX : 1];
#pragma unroll
      for (int i = 0; i < SMAX; ++i)
        if (s0 + i < s1) d[i] = *reinterpret_cast<const uint2 *>(wt + (int64_t)(s0 + i) * 512 + lane * 8);
      uint32_t dw = 0, sh = 0;
      if (tail_here) load_tail<RT>(wt, F, lane, dw, sh);
#pragma unroll
      for (int i = 0; i < SMAX; ++i) {
        const int s = s0 + i;
        if (s < s1) {
          uint32_t pw[20];
          unpack8(d[i], pw);
#pragma unroll
          for (int m = 0; m < 5; ++m) acc = mfma_bf16(pw + 4 * m, lds16(bp + (5 * s + m) * 16), acc);
        }
      }
      if constexpr (RT > 0) {
        if (tail_here) {
          uint32_t pw[16];
          unpack_tail<RT>(dw, sh, pw);
#pragma unroll
          for (int m = 0; m < tail_mfmas(RT); ++m) acc = mfma_bf16(pw + 4 * m, lds16(bp + (5 * F + m) * 16), acc);
        }
      }
    } else {
      for (int s = s0; s < s1; ++s) {
        uint2 d = *reinterpret_cast<const uint2 *>(wt + (int64_t)s * 512 + lane * 8);
        uint32_t pw[20];
        unpack8(d, pw);
#pragma unroll
        for (int m = 0; m < 5; ++m) acc = mfma_bf16(pw + 4 * m, lds16(bp + (5 * s + m) * 16), acc);
      }
      if (tail_here) {
        uint32_t dw = 0, sh = 0, pw[16];
        switch (Rr) {
          case 2:
            load_tail<2>(wt, Fr, lane, dw, sh);
            unpack_tail<2>(dw, sh, pw);
            break;
          case 4:
            load_tail<4>(wt, Fr, lane, dw, sh);
            unpack_tail<4>(dw, sh, pw);
            break;
          default:
            load_tail<6>(wt, Fr, lane, dw, sh);
            unpack_tail<6>(dw, sh, pw);
            break;
        }
        const int tm = (5 * (Rr / 2) + 3) / 4;
        for (int m = 0; m < tm; ++m) acc = mfma_bf16(pw + 4 * m, lds16(bp + (5 * Fr + m) * 16), acc);
      }
    }
  }
  if constexpr (KS > 1) {
    float *red = reinterpret_cast<float *>(smem + 17 * rs);  // [4][64][4]
#pragma unroll
    for (int v = 0; v < 4; ++v) red[(wave * 64 + lane) * 4 + v] = acc[v];
    __syncthreads();
    if (kp != 0) return;
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = 0.f;
    for (int q = 0; q < KS; ++q)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] += red[((wave + q) * 64 + lane) * 4 + v];
  }
  if (!active || n >= cnt) return;
  const int64_t row0 = (int64_t)rt * 16 + 4 * g;
  float *y = a.Y + (t0 + n) * a.ldy;
#pragma unroll
  for (int v = 0; v < 4; ++v)
    if (row0 + v < a.N) y[row0 + v] = (acc[v] * 0.5f) * a.s[row0 + v];
}

// ------------------------------------------------------------------ combine
// One workgroup per token; fixed slot order j = 0..k-1.
__global__ __launch_bounds__(256) void combine_kernel(const float *O, const float *w, const int32_t *pos, int k,
                                                       int H, float *Y, const uint16_t *resid_in,
                                                       uint16_t *resid_out) {
  const int64_t t = blockIdx.x;
  for (int c = threadIdx.x; c < H / 4; c += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int p = pos[t * k + j];
      if (p < 0) continue;
      const float wj = w[t * k + j];
      const float4 o = reinterpret_cast<const float4 *>(O + (int64_t)p * H)[c];
      acc.x = fmaf(wj, o.x, acc.x);
      acc.y = fmaf(wj, o.y, acc.y);
      acc.z = fmaf(wj, o.z, acc.z);
      acc.w = fmaf(wj, o.w, acc.w);
    }
    if (Y) reinterpret_cast<float4 *>(Y + t * H)[c] = acc;
    if (resid_out) {
      const uint2 xi = reinterpret_cast<const uint2 *>(resid_in + t * H)[c];
      const float x0 = __uint_as_float(xi.x << 16), x1 = __uint_as_float(xi.x & 0xFFFF0000u);
      const float x2 = __uint_as_float(xi.y << 16), x3 = __uint_as_float(xi.y & 0xFFFF0000u);
      uint2 r;
      r.x = (uint32_t)f32_to_bf16_rne(x0 + acc.x) | ((uint32_t)f32_to_bf16_rne(x1 + acc.y) << 16);
      r.y = (uint32_t)f32_to_bf16_rne(x2 + acc.z) | ((uint32_t)f32_to_bf16_rne(x3 + acc.w) << 16);
      reinterpret_cast<uint2 *>(resid_out + t * H)[c] = r;
    }
  }
}

// ----------------------------------------------------------------- host side
// Kernels staging more than 64 KiB of LDS must opt in once (gfx950 has 160 KiB).
template <auto Kern>
static int allow_lds(size_t bytes) {
  static bool done = false;  // one flag per kernel instantiation
  if (done || bytes <= 65536) return TMOE_OK;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(Kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)bytes);
  if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute(MaxDynamicSharedMemorySize)");
  done = true;
  return TMOE_OK;
}

int64_t ffn_max_tiles(int64_t pairs, int64_t E) { return cdiv(pairs, 16) + (pairs < E ? pairs : E); }

size_t ffn_ws_bytes(int64_t T, int k, int64_t E, int64_t H, int64_t I) {
  const int64_t P = T * k;
  const Geom gh = make_geom(H), gi = make_geom(I);
  size_t o = 0;
  o = align_up(o + ffn_max_tiles(P, E) * 16, 256);
  o = align_up(o + 16, 256);
  o = align_up(o + (size_t)T * gh.slots * 2, 256);
  o = align_up(o + (size_t)P * I * 4, 256);
  o = align_up(o + (size_t)2 * P * gi.slots * 2, 256);
  o = align_up(o + (size_t)P * 4, 256);
  return o;
}

FfnWs ffn_ws_carve(void *ws, int64_t T, int k, int64_t E, int64_t H, int64_t I) {
  const int64_t P = T * k;
  const Geom gh = make_geom(H), gi = make_geom(I);
  char *b = (char *)ws;
  FfnWs f;
  size_t o = 0;
  f.tiles = (int32_t *)(b + o);
  o = align_up(o + ffn_max_tiles(P, E) * 16, 256);
  f.ntiles = (int32_t *)(b + o);
  o = align_up(o + 16, 256);
  f.xp = (uint16_t *)(b + o);
  o = align_up(o + (size_t)T * gh.slots * 2, 256);
  f.h = (float *)(b + o);
  o = align_up(o + (size_t)P * I * 4, 256);
  f.hp = (uint16_t *)(b + o);
  o = align_up(o + (size_t)2 * P * gi.slots * 2, 256);
  f.hexp = (int32_t *)(b + o);
  return f;
}

template <int F, int RT, int KS>
static int run_gateup(hipStream_t st, const GateUpArgs &a, int64_t max_tiles, int I) {
  const int rs = lds_row_bytes(a.slots);
  size_t lds = (size_t)17 * rs + (KS > 1 ? 4 * 64 * 8 * 4 : 0);
  dim3 grid((unsigned)max_tiles, (unsigned)(I / 16 / (4 / KS)));
  int rc = allow_lds<gateup_kernel<F, RT, KS>>(lds);
  if (rc) return rc;
  hipLaunchKernelGGL((gateup_kernel<F, RT, KS>), grid, dim3(256), lds, st, a);
  TMOE_LAUNCHED("gateup");
  return TMOE_OK;
}

int launch_ffn(hipStream_t st, const tmoe_moe_weights *W, const uint16_t *X, int64_t T, const int32_t *offsets,
               const int32_t *sorted_token, float clamp, float *O, float *Hout, const FfnWs &fw) {
  const int64_t E = W->n_experts, H = W->hidden, I = W->inter, P = T * W->top_k;
  const Geom gh = make_geom(H), gi = make_geom(I);
  if (!(gh.F == 13 && gh.r == 0 && gi.F == 3 && gi.r == 2))
    return fail(TMOE_E_UNSUPPORTED, "expert kernels are built for hidden 2048 and moe_intermediate 512");
  const int64_t max_tiles = ffn_max_tiles(P, E);
  if (max_tiles > 0x7FFFFFFF || T > 0x7FFFFFFF) return fail(TMOE_E_UNSUPPORTED, "too many tokens");
  float *Hn = Hout ? Hout : fw.h;

  hipLaunchKernelGGL(make_tiles_kernel, dim3(1), dim3(256), 0, st, offsets, (int)E, fw.tiles, fw.ntiles);
  TMOE_LAUNCHED("make_tiles");
  hipLaunchKernelGGL(permute_x_kernel, dim3((unsigned)T, (unsigned)cdiv(gh.slots, 256)), dim3(256), 0, st, X, H, T,
                     gh, fw.xp);
  TMOE_LAUNCHED("permute_x");

  GateUpArgs ga;
  ga.gate_p = W->gate_p;
  ga.up_p = W->up_p;
  ga.stride_gu = W->stride_gu;
  ga.gate_s = W->gate_s;
  ga.up_s = W->up_s;
  ga.xp = fw.xp;
  ga.tiles = fw.tiles;
  ga.ntiles = fw.ntiles;
  ga.sorted_token = sorted_token;
  ga.h = Hn;
  ga.I = (int)I;
  ga.slots = gh.slots;
  ga.clamp = clamp;
  int rc = P <= 64 ? run_gateup<13, 0, 4>(st, ga, max_tiles, (int)I) : run_gateup<13, 0, 1>(st, ga, max_tiles, (int)I);
  if (rc) return rc;

  uint16_t *hp_hi = fw.hp, *hp_lo = fw.hp + (size_t)P * gi.slots;
  hipLaunchKernelGGL(permute_h_kernel, dim3((unsigned)P), dim3(256), 0, st, Hn, (int)I, offsets, (int)E, gi, hp_hi,
                     hp_lo, fw.hexp, P);
  TMOE_LAUNCHED("permute_h");

  DownArgs da;
  da.down_p = W->down_p;
  da.stride_d = W->stride_d;
  da.down_s = W->down_s;
  da.hp_hi = hp_hi;
  da.hp_lo = hp_lo;
  da.hexp = fw.hexp;
  da.tiles = fw.tiles;
  da.ntiles = fw.ntiles;
  da.O = O;
  da.H = (int)H;
  da.slots = gi.slots;
  const size_t lds = (size_t)2 * 17 * lds_row_bytes(gi.slots);
  hipLaunchKernelGGL((down_kernel<3, 2>), dim3((unsigned)max_tiles, (unsigned)(H / 64)), dim3(256), lds, st, da);
  TMOE_LAUNCHED("down");
  return TMOE_OK;
}

size_t linear_ws_bytes(int64_t T, int64_t K) { return align_up((size_t)T * make_geom(K).slots * 2, 256); }

template <int F, int RT, int KS>
static int run_linear(hipStream_t st, const LinearArgs &a, int64_t ntok_tiles, int64_t nrt) {
  const int rs = lds_row_bytes(a.slots);
  size_t lds = (size_t)17 * rs + (KS > 1 ? 4 * 64 * 4 * 4 : 0);
  dim3 grid((unsigned)ntok_tiles, (unsigned)cdiv(nrt, 4 / KS));
  int rc = allow_lds<linear_kernel<F, RT, KS>>(lds);
  if (rc) return rc;
  hipLaunchKernelGGL((linear_kernel<F, RT, KS>), grid, dim3(256), lds, st, a);
  TMOE_LAUNCHED("ternary_linear");
  return TMOE_OK;
}

int launch_linear(hipStream_t st, const uint8_t *Pt, const float *s, int64_t N, int64_t K, const uint16_t *X,
                  int64_t ldx, int64_t T, float *Y, int64_t ldy, void *ws) {
  const Geom g = make_geom(K);
  if ((size_t)17 * lds_row_bytes(g.slots) + 4096 > 160 * 1024) return fail(TMOE_E_UNSUPPORTED, "K too large");
  const int64_t nrt = cdiv(N, 16), ntt = cdiv(T, 16);
  if (ntt > 0x7FFFFFFF || nrt > 0x7FFFFFFF) return fail(TMOE_E_UNSUPPORTED, "too large");
  uint16_t *xp = (uint16_t *)ws;
  hipLaunchKernelGGL(permute_x_kernel, dim3((unsigned)T, (unsigned)cdiv(g.slots, 256)), dim3(256), 0, st, X, ldx, T, g,
                     xp);
  TMOE_LAUNCHED("permute_x");
  LinearArgs a;
  a.pt = Pt;
  a.s = s;
  a.xp = xp;
  a.Y = Y;
  a.T = T;
  a.N = N;
  a.ldy = ldy;
  a.slots = g.slots;
  a.g = g;
  const bool small = T <= 16;
  if (g.F == 13 && g.r == 0) return small ? run_linear<13, 0, 4>(st, a, ntt, nrt) : run_linear<13, 0, 1>(st, a, ntt, nrt);
  if (g.F == 3 && g.r == 2) return run_linear<3, 2, 1>(st, a, ntt, nrt);
  return run_linear<-1, 0, 1>(st, a, ntt, nrt);
}

int launch_combine(hipStream_t st, const float *O, const float *w, const int32_t *pos, int64_t T, int k, int64_t H,
                   float *Y, const uint16_t *resid_in, uint16_t *resid_out) {
  if (T > 0x7FFFFFFF) return fail(TMOE_E_UNSUPPORTED, "T too large");
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T), dim3(256), 0, st, O, w, pos, k, (int)H, Y, resid_in, resid_out);
  TMOE_LAUNCHED("combine");
  return TMOE_OK;
}

}  // namespace tmoe
