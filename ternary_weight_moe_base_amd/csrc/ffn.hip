// Ternary GEMV/GEMM kernels on MFMA: the ternary linear, the fused
// gate/up + SiLU/clamp expert half, the down projection, and the combine.
//
// Arithmetic (codeinsider.com.br, "Pesos ternarios": a ternary weight adds,
// subtracts or skips its input; ai.thesatyajit.com, "The shipped code does no
// quantization": an expert computes o = Wd h with h = SiLU(min(g, 7)) times
// clip(u, -7, 7), g = Wg x, u = Wu x):
//  - A trit t enters the matrix core as the 16-bit value 2t, whose bit pattern
//    ((d - 1) mod 4) << 14 (d = t + 1 the base-3 digit) is the same in bf16
//    and fp16: 0xC000 = -2, 0 = 0, 0x4000 = +2. Products with bf16 or fp16
//    operands are exact; MFMA accumulates in fp32; the result is halved.
//  - The tiled layout puts the 8 trits of each MFMA operand slice on 8
//    consecutive input indices, so activations enter the MFMA in their natural
//    order (per row quarter, see Geom).
//  - Digits are decoded two bytes at a time in packed fp16: a byte pair b0, b1
//    becomes the fp16 pair (1024 + b0, 1024 + b1); one packed FMA computes
//    1024 + floor(R / 3) (rounding to the integer grid of [1024, 2048) is the
//    floor), another 1027 + R + floor(R / 3), whose two low bits are
//    (d - 1) mod 4 because d = R - 3 floor(R / 3) == R + floor(R / 3) (mod 4).
//  - gate/up take the bf16 activations directly. The down projection's input h
//    is fp32 (written to the workspace by gate/up). While a down kernel stages
//    a pair's h row it scales the row by a power of two 2^sig that puts the
//    row's largest |h| in [2^14, 2^15), and splits each value into two fp16
//    parts hi = fp16(2^sig h), lo = fp16(2^sig h - hi) (the difference is
//    exact in fp32): hi never overflows, and every value the row's result can
//    feel keeps 22 of its 24 significant bits, for any finite h. Both parts
//    are multiplied exactly on the fp16 matrix cores (the trit operand is the
//    same bit pattern), and the epilogue multiplies the pair's sums by
//    2^-(sig + 1), exactly.
#include "route_util.h"

namespace tmoe {


// ---------------------------------------------------------- trit decoding
__device__ __forceinline__ uint32_t fma16x2(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2, a),
                                                                __builtin_bit_cast(f16x2, b),
                                                                __builtin_bit_cast(f16x2, c)));
}
// v * 2^14 + c per 16-bit half (mod 2^16): moves the two low bits of v to the
// top of the half and adds c. The multiplier passes through an empty asm so
// that the compiler cannot see the power of two (it would emit a shift and an
// add instead of one v_pk_mad_u16).
__device__ __forceinline__ uint32_t mad14x2(uint32_t v, uint32_t c) {
  uint32_t m = 0x40004000u;
  asm("" : "+s"(m));
  const u16x2 x = __builtin_bit_cast(u16x2, v), y = __builtin_bit_cast(u16x2, c), k = __builtin_bit_cast(u16x2, m);
  return __builtin_bit_cast(uint32_t, (u16x2)(x * k + y));
}

// fp16 constants (two copies per dword)
#define K_THIRD 0x35553555u  // 0.333251953125
#define K_C1 0x61556155u     // 682.5

// Five pair-words (digits q = 0..4 of both bytes) from v = fp16 (1024 + b0, 1024 + b1).
// With v_q = 1024 + R_q, the chain FMA v_(q+1) = fp16(K_THIRD v_q + 682.5) is
// 1023.75 + R_q / 3 - 8e-5 R_q before rounding, so fp16's integer grid on
// [1024, 2048) rounds it to 1024 + R_(q+1), R_(q+1) = floor(R_q / 3); hence
// the bit patterns of v_q and v_(q+1) sum to 0xC800 + R_q + R_(q+1) =
// 0xC800 + 4 R_(q+1) + d_q, and 2^14 (v_q + v_(q+1) + 3) mod 2^16 is
// ((d_q + 3) mod 4) << 14: 0xC000, 0, 0x4000 for d = 0, 1, 2, the bf16 and
// fp16 bit pattern of 2t. Per digit: one chain FMA, one integer multiply-add
// for (v_(q+1) + 3) << 14, one for the operand.
__device__ __forceinline__ void digits5(uint32_t v, uint32_t *pw) {
  uint32_t c[5];
  c[0] = v;
#pragma unroll
  for (int q = 1; q < 5; ++q) c[q] = fma16x2(c[q - 1], K_THIRD, K_C1);
  uint32_t hi = mad14x2(c[4], 0xC000C000u);  // (v_4 + 3) << 14: the top digit's operand
  pw[4] = hi;
#pragma unroll
  for (int q = 3; q >= 0; --q) {
    pw[q] = mad14x2(c[q], hi);
    if (q > 0) hi = mad14x2(c[q], 0xC000C000u);
  }
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


// Workgroups of a batched gate/up or down grid that walks its items (two per
// CU: the staged activations take 71 KB of LDS). With few pairs per expert
// most of the worst-case tiles do not exist, and walking saves launching
// them (T = 64: 69.5 -> 66.4 us per layer); with many, one workgroup per item
// balances better.
constexpr int kWalkWgs = 512;
__host__ inline unsigned walk_grid(int64_t items_max, bool walk) {
  return (unsigned)(walk && items_max > kWalkWgs ? kWalkWgs : items_max);
}

// 8 bytes of a weight tile, loaded non-temporally. With few pairs per expert
// (decode, small batches) each weight tile is read once per call, and such
// loads keep the stream from displacing the activations, logits and routing
// data held in the caches (measured: 3% faster decode); with many tiles per
// expert (prefill) the cached re-reads win and plain loads are used.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ldw8(const uint8_t *p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
  return make_uint2(v[0], v[1]);
}

// LDS row stride (bytes) of a staged operand row with `slots` 16-bit values:
// slots/2 = 16M dwords; +4 dwords makes the 16 token rows start in 16
// different 4-bank groups of the 64 LDS banks.
__host__ __device__ inline int lds_row_bytes(int slots) { return slots * 2 + 16; }

// ------------------------------------------------------------- staging
// Operand row n of LDS <- input row `src` (16-bit values): position g*QS + j
// holds src[5Qg + j] for j < 5Q and 5Qg + j < K, zero otherwise.
__device__ inline void stage_row(char *dst, const uint16_t *src, const Geom &g, int tid, int nthreads) {
  for (int i = tid; i < g.slots; i += nthreads) {
    const int quarter = i / g.QS, j = i - quarter * g.QS;
    const int64_t k = operand_k(g, quarter, j);
    reinterpret_cast<uint16_t *>(dst)[i] = k >= 0 ? src[k] : (uint16_t)0;
  }
}

__device__ inline void zero_row(char *dst, int slots, int tid, int nthreads) {
  for (int c = tid; c < slots / 8; c += nthreads) *reinterpret_cast<uint4 *>(dst + c * 16) = make_uint4(0, 0, 0, 0);
}

// ---------------------------------------------------------------- tiles
// Work tiles of up to TILE grouped pairs of one expert, in expert order.
template <int TILE>
__global__ __launch_bounds__(256) void make_tiles_kernel(const int32_t *offsets, int E, int32_t *tiles,
                                                          int32_t *ntiles) {
  __shared__ int nt[1024];
  __shared__ int tmp[256];
  for (int e = threadIdx.x; e < E; e += 256) nt[e] = (offsets[e + 1] - offsets[e] + TILE - 1) / TILE;
  __syncthreads();
  int total = block_exclusive_scan<256>(nt, E, tmp);
  for (int e = threadIdx.x; e < E; e += 256) {
    int c = offsets[e + 1] - offsets[e], base = nt[e];
    for (int i = 0; TILE * i < c; ++i) {
      int4 tv = make_int4(e, offsets[e] + TILE * i, min(TILE, c - TILE * i), 0);
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
  const uint16_t *X;  // [T][H] bf16, natural order
  const int32_t *tiles, *ntiles, *sorted_token;
  float *h;            // [pairs][I] fp32 (grouped order) or null: a copy of h for the caller
  float *hf;           // [pairs][I] fp32 h in grouped order (the down projection's input)
  uint32_t *hmax;      // [pairs][kTbMaxGroups] largest |h| (fp32 bits) per row group (token-blocked path)
  Geom gx, gd;         // operand geometry of gate/up (K = H) and of down (K = I)
  int I;
  float clamp;
  const int32_t *offsets;  // [E+1] grouping offsets (token-blocked kernel)
  // routing prologue (decode path only)
  DecodeRoute r;
  int T, E, k;
};

__device__ inline uint32_t store_h4(const GateUpArgs &a, int64_t p, int row0, const f32x4 &gs, const f32x4 &us,
                                    const float4 &sg, const float4 &su, bool store = true) {
  const float sgv[4] = {sg.x, sg.y, sg.z, sg.w}, suv[4] = {su.x, su.y, su.z, su.w};
  const float c = a.clamp;
  float hv[4];
  uint32_t mx = 0u;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float gg = (gs[v] * 0.5f) * sgv[v];
    const float uu = (us[v] * 0.5f) * suv[v];
    const float z = fminf(gg, c);
    hv[v] = __fdividef(z, 1.f + __expf(-z)) * fminf(fmaxf(uu, -c), c);
    mx = max(mx, __float_as_uint(hv[v]) & 0x7FFFFFFFu);
  }
  if (store) {
    const float4 h4 = make_float4(hv[0], hv[1], hv[2], hv[3]);
    *reinterpret_cast<float4 *>(a.hf + p * a.I + row0) = h4;
    if (a.h) *reinterpret_cast<float4 *>(a.h + p * a.I + row0) = h4;
  }
  return mx;
}

constexpr int kTbMaxGroupsH = 4;  // row groups per pair in the gate/up's hmax (kTbMaxGroups)

// ------------------------------------------------ down operand staging
// The h rows of `cnt` grouped pairs (fp32, row n at h + n * I) become the down
// projection's operand in LDS: two fp16 planes (row n of plane q at
// pl[q] + n * rs) in the operand layout (position g * 8M + j holds input
// 5Qg + j, zero where no input is held). Row n is scaled by 2^sig[n], sig
// chosen so that the row's largest |h| lies in [2^14, 2^15) (sig = 0 for an
// all-zero or non-finite row): hi = fp16(2^sig h) then never overflows, and
// lo = fp16(2^sig h - hi) keeps the next 11 bits; values below 2^-28 of the
// row's largest only lose bits under 2^-39 of it. Wavefront w of NW takes rows
// w, w + NW, ... (at most RPW each), RB rows at a time: the loads of a batch
// are all issued before its first row is reduced.
template <int NW, int RPW, int M, int RB = RPW>
__device__ inline void stage_h_parts(const float *h, int cnt, int I, int q5, char *pl0, char *pl1, int rs, int *sig) {
  static_assert(RPW % RB == 0, "whole batches");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NCH = 4 * M;            // 16-byte chunks (8 positions) per staged row
  constexpr int NPL = (NCH + 63) / 64;  // chunks per lane
#pragma unroll
  for (int b0 = 0; b0 < RPW; b0 += RB) {
    if (wave + NW * b0 >= cnt) break;
    float v[RB][NPL][8];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int n = wave + NW * (b0 + i);
#pragma unroll
      for (int u = 0; u < NPL; ++u) {
        const int c = lane + 64 * u;
        const int quarter = c / M, j0 = 8 * (c - quarter * M), k0 = q5 * quarter + j0;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          // q5, I and k0 are even, so both values of a pair are inputs or neither is
          float2 f = make_float2(0.f, 0.f);
          if (n < cnt && c < NCH && j0 + e < q5 && k0 + e < I)
            f = *reinterpret_cast<const float2 *>(h + (int64_t)n * I + k0 + e);
          v[i][u][e] = f.x;
          v[i][u][e + 1] = f.y;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int n = wave + NW * (b0 + i);
      if (n >= cnt) break;
      uint32_t mx = 0;
#pragma unroll
      for (int u = 0; u < NPL; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = max(mx, __float_as_uint(v[i][u][e]) & 0x7FFFFFFFu);
      mx = wave_max_u32(mx);
      int sg = 0;
      if (mx != 0 && mx < 0x7F800000u) {
        int ex;
        (void)frexpf(__uint_as_float(mx), &ex);  // largest |h| = f 2^ex, f in [1/2, 1)
        sg = 15 - ex;
      }
#pragma unroll
      for (int u = 0; u < NPL; ++u) {
        const int c = lane + 64 * u;
        if (c >= NCH) continue;
        uint32_t w[2][4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float a0 = ldexpf(v[i][u][e], sg), a1 = ldexpf(v[i][u][e + 1], sg);
          const _Float16 h0 = (_Float16)a0, h1 = (_Float16)a1;
          const _Float16 l0 = (_Float16)(a0 - (float)h0), l1 = (_Float16)(a1 - (float)h1);
          w[0][e >> 1] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
          w[1][e >> 1] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
        }
        *reinterpret_cast<uint4 *>(pl0 + n * rs + c * 16) = make_uint4(w[0][0], w[0][1], w[0][2], w[0][3]);
        *reinterpret_cast<uint4 *>(pl1 + n * rs + c * 16) = make_uint4(w[1][0], w[1][1], w[1][2], w[1][3]);
      }
      if (lane == 0) sig[n] = sg;
    }
  }
}

// The same operand staging when each row's largest |h| is already known (the
// token-blocked gate/up writes it per row group, hmax[row][q] for q <
// ngroups): every thread takes whole 16-byte chunks of any rows, all of its
// loads in flight at once, with no reduction across lanes. after_loads() runs
// once the h loads are issued (its own loads then queue behind them).
template <int NT, int M, class AfterLoads>
__device__ inline void stage_h_known(const float *h, const uint32_t *hmax, int ngroups, int cnt, int I, int q5,
                                     char *pl0, char *pl1, int rs, int *sig, AfterLoads after_loads) {
  constexpr int NCH = 4 * M;                    // 16-byte chunks per staged row
  constexpr int PER = (64 * NCH + NT - 1) / NT;  // chunks per thread (at most 64 rows)
  // the thread index through an empty asm: a caller that stages inside a loop
  // must not have the chunk offsets derived from it hoisted out of the loop
  // and held in registers across its products
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  for (int r = tid; r < cnt; r += NT) {
    uint32_t mx = 0u;
    for (int q = 0; q < ngroups; ++q) mx = max(mx, hmax[(int64_t)r * kTbMaxGroupsH + q]);
    int sg = 0;
    if (mx != 0 && mx < 0x7F800000u) {
      int ex;
      (void)frexpf(__uint_as_float(mx), &ex);
      sg = 15 - ex;
    }
    sig[r] = sg;
  }
  float v[PER][8];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = tid + NT * u, row = i / NCH, c = i - row * NCH;
    const int quarter = c / M, j0 = 8 * (c - quarter * M), k0 = q5 * quarter + j0;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float2 f = make_float2(0.f, 0.f);
      if (row < cnt && j0 + e < q5 && k0 + e < I) f = *reinterpret_cast<const float2 *>(h + (int64_t)row * I + k0 + e);
      v[u][e] = f.x;
      v[u][e + 1] = f.y;
    }
  }
  after_loads();
  __syncthreads();  // sig[] written
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = tid + NT * u, row = i / NCH, c = i - row * NCH;
    if (row >= cnt) continue;
    const int sg = sig[row];
    uint32_t w[2][4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float a0 = ldexpf(v[u][e], sg), a1 = ldexpf(v[u][e + 1], sg);
      const _Float16 h0 = (_Float16)a0, h1 = (_Float16)a1;
      const _Float16 l0 = (_Float16)(a0 - (float)h0), l1 = (_Float16)(a1 - (float)h1);
      w[0][e >> 1] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
      w[1][e >> 1] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
    }
    *reinterpret_cast<uint4 *>(pl0 + row * rs + c * 16) = make_uint4(w[0][0], w[0][1], w[0][2], w[0][3]);
    *reinterpret_cast<uint4 *>(pl1 + row * rs + c * 16) = make_uint4(w[1][0], w[1][1], w[1][2], w[1][3]);
  }
}

// ------------------------------------------------------ routing prologue
// Decode path (T <= 16 tokens, so one work tile per hit expert): every
// workgroup certifies the top-k of all tokens from the fp64 logits (one
// wavefront per token; the double-double recompute when the bound cannot
// separate the top k+1), then each (token, slot) pair finds, from the others,
// its grouped position (pairs of lower experts, then of the same expert and a
// lower token) and its tile (hit experts below its expert). The workgroup takes
// the blockIdx.x-th hit expert (in expert order) as its tile. Workgroup (0, 0)
// publishes idx, w, pos, the grouped tokens, slots and weights, and the tiles.
struct RouteLds {
  int32_t sidx[kDecodeMaxT * 16];
  float sw[kDecodeMaxT * 16];
  uint32_t hit[32];  // bit e: some token chose expert e (E <= 1024)
  int32_t tok[kDecodeMaxT];
  int32_t info[3];  // expert (-1: none), start, count of this workgroup's tile
  int32_t nfix;
};

// largest of a lane's bound slots (fp64 bits of values >= 0 order as integers)
__device__ inline uint64_t slot_max(const uint64_t (&v)[kRouterMaxSlots / 64]) {
  uint64_t m = v[0];
#pragma unroll
  for (int u = 1; u < kRouterMaxSlots / 64; ++u) m = m > v[u] ? m : v[u];
  return m;
}

template <int NPL>
__device__ inline void route_prologue(const GateUpArgs &a, RouteLds &s, char *smem, int rs) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const DecodeRoute &r = a.r;
  const int T = a.T, E = a.E, k = a.k, P = T * k;
  const bool publish = blockIdx.x == 0 && blockIdx.y == 0;
  // every token's activations (2048 inputs = 4 KB, operand order = natural
  // order) into LDS row t by direct buffer loads, issued first: wavefront w
  // copies the w-th KB of each row. The buffer range bounds every read.
  {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    for (int t = 0; t < T; ++t) {
      const __amdgpu_buffer_rsrc_t row =
          __builtin_amdgcn_make_buffer_rsrc((void *)(a.X + (int64_t)t * 2048), (short)0, 4096, kBufWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          row, (__attribute__((address_space(3))) void *)(smem + t * rs + wv * 1024), 16, lane * 16 + wv * 1024, 0, 0,
          0);
    }
  }
  // logits and bound slots of this wavefront's tokens (t = wave + 4q; only
  // read for t < T), in flight with the staging below. No load has an
  // alternative value merged with it (indices are clamped, duplicate slots are
  // harmless to a maximum, logits past E are replaced after arrival): a load
  // merged with another value at a branch makes the compiler wait for it
  // there, one round trip per load.
  double lv[kDecodeMaxT / 4][NPL];
  uint64_t bs[kDecodeMaxT / 4][kRouterMaxSlots / 64];
#pragma unroll
  for (int q = 0; q < kDecodeMaxT / 4; ++q) {
    const int t = wave + 4 * q;
    if (t < T) {
      const double *lg = r.lg + (int64_t)t * E;
#pragma unroll
      for (int j = 0; j < NPL; ++j) lv[q][j] = lg[min(lane * NPL + j, E - 1)];
      const uint64_t *slots = r.bnd + (int64_t)t * r.nb;
#pragma unroll
      for (int u = 0; u < kRouterMaxSlots / 64; ++u) bs[q][u] = slots[min(lane + 64 * u, r.nb - 1)];
    }
  }
  // padding inputs 2048..2079 of the token rows and the zero row 16
  const int nc = a.gx.slots / 8;
  for (int i = threadIdx.x; i < T * (nc - 256); i += 256)
    *reinterpret_cast<uint4 *>(smem + (i / (nc - 256)) * rs + (256 + i % (nc - 256)) * 16) = make_uint4(0, 0, 0, 0);
  zero_row(smem + 16 * rs, a.gx.slots, threadIdx.x, 256);
  if (threadIdx.x < 32) s.hit[threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    s.info[0] = -1;
    s.nfix = 0;
  }
  TMOE_WAIT_VM(0);  // the activation rows and the routing loads above
  // the slot maxima are formed only now (otherwise the compiler reduces each
  // token's slots right after their loads, waiting there token by token)
#pragma unroll
  for (int q = 0; q < kDecodeMaxT / 4; ++q)
    if (wave + 4 * q < T)
#pragma unroll
      for (int u = 0; u < kRouterMaxSlots / 64; ++u) asm volatile("" : "+v"(bs[q][u]));
  lds_barrier();
  if (T == 1) {
    // one token: wavefront 0 selects its k experts; their ranks among the k
    // (all distinct) are the grouped positions and the tile indices
    if (wave == 0) {
      const double B = r.bscale * bitsd(wave_max_u64(slot_max(bs[0])));
#pragma unroll
      for (int j = 0; j < NPL; ++j) lv[0][j] = lane * NPL + j < E ? lv[0][j] : 0.0;
      int nfix = 0;
      if (!topk_certified_v<NPL, true>(lv[0], r.lg, E, k, B, s.sidx, s.sw)) {
        nfix = 1;
        topk_dd<NPL>(a.X, (int)a.gx.K, r.Wr, r.bias, E, k, s.sidx, s.sw, nullptr);
      }
      const int e = lane < k ? s.sidx[lane] : 0x7FFFFFFF;
      const float wv = lane < k ? s.sw[lane] : 0.f;
      int rank = 0;
      for (int j = 0; j < k; ++j) rank += __builtin_amdgcn_readlane(e, j) < e;
      if (lane < k && rank == (int)blockIdx.x) {
        s.tok[0] = 0;
        s.info[1] = rank;
        s.info[2] = 1;
        s.info[0] = e;
      }
      if (publish) {
        if (lane < k) {
          r.idx[lane] = e;
          r.w[lane] = wv;
          r.pos[lane] = rank;
          r.sorted_token[rank] = 0;
          r.sorted_slot[rank] = lane;
          r.pair_w[rank] = wv;
          reinterpret_cast<int4 *>(r.tiles)[rank] = make_int4(e, rank, 1, 0);
        }
        if (lane == 0) {
          *r.ntiles = k;
          if (r.n_fixup) *r.n_fixup = nfix;
        }
      }
    }
    lds_barrier();  // the published stores need not land before the expert work starts
    return;
  }
#pragma unroll
  for (int q = 0; q < kDecodeMaxT / 4; ++q) {
    const int t = wave + 4 * q;
    if (t < T) {
      const double B = r.bscale * bitsd(wave_max_u64(slot_max(bs[q])));
#pragma unroll
      for (int j = 0; j < NPL; ++j) lv[q][j] = lane * NPL + j < E ? lv[q][j] : 0.0;
      if (!topk_certified_v<NPL, true>(lv[q], r.lg + (int64_t)t * E, E, k, B, s.sidx + t * k, s.sw + t * k)) {
        if (lane == 0) atomicAdd(&s.nfix, 1);
        topk_dd<NPL>(a.X + (int64_t)t * a.gx.K, (int)a.gx.K, r.Wr, r.bias, E, k, s.sidx + t * k, s.sw + t * k,
                     nullptr);
      }
    }
  }
  __syncthreads();
  const int i = threadIdx.x;
  if (i < P) atomicOr(&s.hit[s.sidx[i] >> 5], 1u << (s.sidx[i] & 31));
  __syncthreads();
  if (i < P) {
    const int t = i / k, j = i - t * k, e = s.sidx[i];
    int before = 0, same = 0, cnt = 0;
    for (int i2 = 0; i2 < P; ++i2) {
      const int e2 = s.sidx[i2];
      before += e2 < e;
      if (e2 == e) {
        ++cnt;
        same += i2 < i;  // same expert, lower token
      }
    }
    const int pos = before + same;
    int tl = __popc(s.hit[e >> 5] & ((1u << (e & 31)) - 1u));
    for (int q = 0; q < (e >> 5); ++q) tl += __popc(s.hit[q]);
    if (tl == (int)blockIdx.x) {
      s.tok[same] = t;
      if (same == 0) {
        s.info[1] = before;
        s.info[2] = cnt;
        s.info[0] = e;
      }
    }
    if (publish) {
      r.idx[i] = e;
      r.w[i] = s.sw[i];
      r.pos[i] = pos;
      r.sorted_token[pos] = t;
      r.sorted_slot[pos] = j;
      r.pair_w[pos] = s.sw[i];
      if (same == 0) reinterpret_cast<int4 *>(r.tiles)[tl] = make_int4(e, before, cnt, 0);
    }
  }
  if (publish && threadIdx.x == 0) {
    int nh = 0;
    for (int q = 0; q < (E + 31) / 32; ++q) nh += __popc(s.hit[q]);
    *r.ntiles = nh;
    if (r.n_fixup) *r.n_fixup = s.nfix;
  }
  lds_barrier();
}

// SiLU with the hardware exponential and a fast divide (a few ulp in fp32)
__device__ __forceinline__ float silu(float z) { return __fdividef(z, 1.f + __expf(-z)); }

// h = SiLU(min(g, c)) * clip(u, -c, c) of four consecutive intermediate rows
// row0 .. row0+3 of grouped pair p, from the gate / up sums (trits entered as
// 2t) and the row scales; stored as fp32 in grouped order (one 16-byte store),
// and into the caller's copy if requested.
struct GateUpArgs;
__device__ inline uint32_t store_h4(const GateUpArgs &a, int64_t p, int row0, const f32x4 &gs, const f32x4 &us,
                                    const float4 &sg, const float4 &su, bool store);

// Workgroup = 4 wavefronts. KS wavefronts split the K steps of one 16-row tile
// (partial sums reduced in LDS in fixed order); with KS = 1 each wavefront
// takes R row tiles and reads every activation slice from LDS once for all of
// them (and for both matrices). blockIdx.x = work tile (expert, <= 16 pairs),
// blockIdx.y = group of (4 / KS) * R row tiles.
// RNPL > 0: decode path with the routing prologue (experts per lane of its top-k).
template <int F, int RT, int KS, int RNPL, int R, int NW>
__device__ inline void gateup_work(const GateUpArgs &a, char *smem, int tile_id, int ry) {
  static_assert(KS == 1 || R == 1, "row tiles per wavefront need the full K range");
  static_assert(NW == 4 || (KS == 1 && RNPL == 0), "eight wavefronts only on the batched full-K path");
  int e, start, cnt;
  const int32_t *toks;
  const int rs0 = lds_row_bytes(a.gx.slots);
  if constexpr (RNPL > 0) {
    static_assert(F == 13 && RT == 0, "the prologue copies activation rows as 2048 inputs");
    __shared__ RouteLds rl;
    route_prologue<RNPL>(a, rl, smem, rs0);
    e = rl.info[0];
    if (e < 0) return;
    start = rl.info[1];
    cnt = rl.info[2];
    toks = rl.tok;
  } else {
    const int tile = tile_id;
    const int4 td = reinterpret_cast<const int4 *>(a.tiles)[tile];
    e = __builtin_amdgcn_readfirstlane(td.x);
    start = __builtin_amdgcn_readfirstlane(td.y);
    cnt = __builtin_amdgcn_readfirstlane(td.z);
    toks = a.sorted_token + start;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int RTB = NW / KS;
  constexpr int M = 5 * F + tail_mfmas(RT);
  constexpr int SMAX = (F + KS - 1) / KS;
  const int rtb = ry * RTB * R + wave / KS;  // row tiles rtb + RTB r
  const int kp = wave % KS;
  const int rs = lds_row_bytes(a.gx.slots);
  char *xs = smem;  // [17][rs]; row 16 = zeros

  if constexpr (RNPL == 0) {
    // Activations of the tile's pairs (natural order = operand order for
    // H = 2048), by buffer loads straight into LDS issued before the weights:
    // loads complete in issue order, so the wait for these leaves the weights
    // in flight, and each K step below waits only for its own weights. (The
    // flat-encoded global form would make the compiler wait for every load
    // before the first product.) Wavefront w copies rows w, w + NW, ...; each
    // row is four 1 KB slices (the padding inputs 2048..2079 were cleared at
    // launch). The buffer resource's 4096-byte range bounds every read.
    static_assert(16 % NW == 0, "rows per wavefront");
    const int tokv = (lane & 15) < cnt ? toks[lane & 15] : 0;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    int tks[16 / NW];
#pragma unroll
    for (int j = 0; j < 16 / NW; ++j) tks[j] = __builtin_amdgcn_readlane(tokv, wv + NW * j);
#pragma unroll
    for (int j = 0; j < 16 / NW; ++j) {
      const int nrow = wv + NW * j;
      if (nrow < cnt) {
        const int tk = tks[j];
        const __amdgpu_buffer_rsrc_t row =
            __builtin_amdgcn_make_buffer_rsrc((void *)(a.X + (int64_t)tk * 2048), (short)0, 4096, kBufWord3);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              row, (__attribute__((address_space(3))) void *)(xs + nrow * rs + c * 1024), 16, lane * 16 + c * 1024, 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // the weight loads stay behind these
  }

  // then the weights: all loads of this wavefront are in flight while x lands
  const int64_t tbytes = 64 * (int64_t)(8 * F + RT);
  const int s0 = kp * F / KS, s1 = (kp + 1) * F / KS;
  const bool tail_here = RT > 0 && kp == KS - 1;
  uint2 gd[R][SMAX], ud[R][SMAX];
  uint32_t gdw[R], gsh[R], udw[R], ush[R];
  float4 sg[R], su[R];
  // issued in the order the K steps consume them, so step 0 can start while
  // later steps are still arriving
#pragma unroll
  for (int i = 0; i < SMAX; ++i) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t off = (int64_t)e * a.stride_gu + (int64_t)(rtb + RTB * r) * tbytes + (int64_t)(s0 + i) * 512;
      if (s0 + i < s1) {
        gd[r][i] = ldw8(a.gate_p + off + lane * 8);
        ud[r][i] = ldw8(a.up_p + off + lane * 8);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rt = rtb + RTB * r;
    const uint8_t *gt = a.gate_p + (int64_t)e * a.stride_gu + (int64_t)rt * tbytes;
    const uint8_t *ut = a.up_p + (int64_t)e * a.stride_gu + (int64_t)rt * tbytes;
    gdw[r] = gsh[r] = udw[r] = ush[r] = 0;
    if (tail_here) {
      load_tail<RT>(gt, F, lane, gdw[r], gsh[r]);
      load_tail<RT>(ut, F, lane, udw[r], ush[r]);
    }
    // row scales of this lane's four output rows (epilogue), fetched with the weights
    const int row0 = rt * 16 + 4 * (lane >> 4);
    sg[r] = *reinterpret_cast<const float4 *>(a.gate_s + (int64_t)e * a.I + row0);
    su[r] = *reinterpret_cast<const float4 *>(a.up_s + (int64_t)e * a.I + row0);
  }

  if constexpr (RNPL == 0) {
    // every wavefront has at least 2 (F / KS) R weight loads behind its copies
    __builtin_amdgcn_sched_barrier(0);
    TMOE_WAIT_VM(2 * (F / KS) * R);
    __builtin_amdgcn_s_barrier();
  }
  // (with the routing prologue the activations were staged before its last barrier)

  const int n = lane & 15, g = lane >> 4;
  const int brow = n < cnt ? (RNPL > 0 ? toks[n] : n) : 16;
  const char *bp = xs + brow * rs + g * M * 16;
  f32x4 accg[R], accu[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    accg[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    accu[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < SMAX; ++i) {
    const int s = s0 + i;
    if (s < s1) {
      u32x4 bx[5];
#pragma unroll
      for (int m = 0; m < 5; ++m) bx[m] = lds16(bp + (5 * s + m) * 16);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        uint32_t pg[20], pu[20];
        unpack8(gd[r][i], pg);
        unpack8(ud[r][i], pu);
#pragma unroll
        for (int m = 0; m < 5; ++m) {
          accg[r] = mfma_bf16(pg + 4 * m, bx[m], accg[r]);
          accu[r] = mfma_bf16(pu + 4 * m, bx[m], accu[r]);
        }
      }
    }
  }
  if constexpr (RT > 0) {
    if (tail_here) {
      u32x4 bx[tail_mfmas(RT)];
#pragma unroll
      for (int m = 0; m < tail_mfmas(RT); ++m) bx[m] = lds16(bp + (5 * F + m) * 16);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        uint32_t pg[16], pu[16];
        unpack_tail<RT>(gdw[r], gsh[r], pg);
        unpack_tail<RT>(udw[r], ush[r], pu);
#pragma unroll
        for (int m = 0; m < tail_mfmas(RT); ++m) {
          accg[r] = mfma_bf16(pg + 4 * m, bx[m], accg[r]);
          accu[r] = mfma_bf16(pu + 4 * m, bx[m], accu[r]);
        }
      }
    }
  }
  if constexpr (KS > 1) {
    static_assert(KS == 4, "the K split is four wavefronts");
    float *red = reinterpret_cast<float *>(smem + 17 * rs);  // [4 waves][64 lanes][8]
    float *mine = red + (wave * 64 + lane) * 8;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      mine[v] = accg[0][v];
      mine[4 + v] = accu[0][v];
    }
    __syncthreads();
    // wavefront w finishes row 4g + w of every lane's column (partials summed in wave order)
    const int v = wave;
    float gs = 0.f, us = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      gs += red[(q * 64 + lane) * 8 + v];
      us += red[(q * 64 + lane) * 8 + 4 + v];
    }
    if (n >= cnt) return;
    const float sgv[4] = {sg[0].x, sg[0].y, sg[0].z, sg[0].w}, suv[4] = {su[0].x, su[0].y, su[0].z, su[0].w};
    const float c = a.clamp;
    const float gg = (gs * 0.5f) * sgv[v];
    const float uu = (us * 0.5f) * suv[v];
    const float hv = silu(fminf(gg, c)) * fminf(fmaxf(uu, -c), c);
    const int nn = rtb * 16 + 4 * g + v;
    const int64_t p = start + n;
    a.hf[p * a.I + nn] = hv;
    if (a.h) a.h[p * a.I + nn] = hv;
    return;
  }
  if (n >= cnt) return;
  const int64_t p = start + n;
#pragma unroll
  for (int r = 0; r < R; ++r) store_h4(a, p, (rtb + RTB * r) * 16 + 4 * g, accg[r], accu[r], sg[r], su[r], true);
}

// Decode (RNPL > 0): the grid is (hit experts, row-tile groups). Otherwise the
// grid is a fixed number of workgroups that walk the (work tile, row-tile
// group) items, so no workgroup is launched for a tile that does not exist.
template <int F, int RT, int KS, int RNPL, int R, int NW>
__global__ __launch_bounds__(64 * NW) void gateup_kernel(GateUpArgs a) {
  extern __shared__ __align__(16) char smem[];
  if constexpr (RNPL > 0) {
    gateup_work<F, RT, KS, RNPL, R, NW>(a, smem, blockIdx.x, blockIdx.y);
  } else {
    static_assert(F == 13 && RT == 0, "activation rows are copied as 2048 inputs");
    // padding inputs 2048..2079 of the 16 token rows, and the zero row 16
    const int rs = lds_row_bytes(a.gx.slots), nc = a.gx.slots / 8;
    for (int i = threadIdx.x; i < 16 * (nc - 256) + nc; i += 64 * NW) {
      const int row = i < 16 * (nc - 256) ? i / (nc - 256) : 16;
      const int c = row < 16 ? 256 + i % (nc - 256) : i - 16 * (nc - 256);
      *reinterpret_cast<uint4 *>(smem + row * rs + c * 16) = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
    const int groups = a.I / 16 / (NW / KS) / R;
    const int nitems = *a.ntiles * groups;
    for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
      const int tile = item / groups;
      gateup_work<F, RT, KS, RNPL, R, NW>(a, smem, tile, item - tile * groups);
      __syncthreads();  // the staged activations are reused by the next item
    }
  }
}

// ------------------------------------------- token-blocked work items
// Work item of a token-blocked kernel: a 64-pair block and a row group. The
// grid is 1-D, 8 * groups * ceil(max blocks / 8) workgroups; the dispatcher
// hands consecutive workgroups to the eight XCDs in turn, so XCD x runs
// workgroups x, x + 8, x + 16, ... It gets blocks x * per .. x * per + per - 1
// (per = ceil(nblk / 8)) in order, the row groups of each block one after
// another: the row groups of a block (the same activations) and the blocks of
// one expert (the same weights) run on one XCD close together in time and
// share its L2. blk = nblk: no work.
struct TbItem {
  int blk, grp;
};
__device__ __forceinline__ TbItem tb_item(int nblk, int groups) {
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int per = (nblk + 7) >> 3;
  const int b = j / groups;
  TbItem it;
  it.grp = j - b * groups;
  it.blk = b < per ? min(x * per + b, nblk) : nblk;
  return it;
}
// workgroups of a token-blocked launch
static inline unsigned tb_grid(int64_t max_blocks, int groups) {
  return (unsigned)(8 * groups * ((max_blocks + 7) / 8));
}

// ------------------------------------------- gate / up, token-blocked
// Many pairs per expert (prefill): a workgroup takes a block of up to 64 pairs
// of one expert and 256 intermediate rows (eight wavefronts, two row tiles
// each). Each wavefront decodes the weights of a K step once for its two row
// tiles and applies them to all four token tiles, and each activation slice it
// reads from LDS feeds both row tiles, so a product costs 1/2 of an LDS read
// and 1/4 of a decode. Activations stream through LDS one K step at a time by
// direct global-to-LDS loads, kTbDepth - 1 steps ahead; a step's buffer is
// [token tile][slice m][quarter g][column n] x 16 B, so the 16 columns of an
// operand read are consecutive (no bank conflicts). Inputs past K are read
// from a valid address (their trits are zero). Weights stream kTbWDepth steps
// ahead of their use. The epilogue also writes, per pair, the largest |h| of
// the workgroup's rows (hmax[pair][row group]), which the down projection
// uses to pick the pair's scale.
constexpr int kTbWaves = 8, kTbR = 2, kTbDepth = 4, kTbWDepth = 3, kTbStepBytes = 4 * 5 * 64 * 16;
constexpr int kTbRows = 16 * kTbWaves * kTbR;  // intermediate rows per workgroup
constexpr int kTbMaxGroups = kTbMaxGroupsH;   // row groups per pair kept in hmax

// s_waitcnt vmcnt(n) for a value known only after unrolling (0 <= n <= 31)
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define TMOE_VM_CASE(k) case k: TMOE_WAIT_VM(k); break;
    TMOE_VM_CASE(0) TMOE_VM_CASE(1) TMOE_VM_CASE(2) TMOE_VM_CASE(3) TMOE_VM_CASE(4) TMOE_VM_CASE(5)
    TMOE_VM_CASE(6) TMOE_VM_CASE(7) TMOE_VM_CASE(8) TMOE_VM_CASE(9) TMOE_VM_CASE(10) TMOE_VM_CASE(11)
    TMOE_VM_CASE(12) TMOE_VM_CASE(13) TMOE_VM_CASE(14) TMOE_VM_CASE(15) TMOE_VM_CASE(16) TMOE_VM_CASE(17)
    TMOE_VM_CASE(18) TMOE_VM_CASE(19) TMOE_VM_CASE(20) TMOE_VM_CASE(21) TMOE_VM_CASE(22) TMOE_VM_CASE(23)
    TMOE_VM_CASE(24) TMOE_VM_CASE(25) TMOE_VM_CASE(26) TMOE_VM_CASE(27) TMOE_VM_CASE(28) TMOE_VM_CASE(29)
    TMOE_VM_CASE(30)
#undef TMOE_VM_CASE
    default: TMOE_WAIT_VM(0); break;
  }
}

// Vector-memory loads issued after step s's activation loads, at the wait of
// step s. Issue order: prologue W(0..kTbWDepth-1), A(0..kTbDepth-2); then in
// step i: W(i + kTbWDepth), the wait and the barrier, A(i + kTbDepth - 1),
// each while it exists. A(s) = nj loads, W(s) = 2 kTbR loads.
__device__ __forceinline__ int tb_after_act(int s, int nj, int F) {
  constexpr int WL = 2 * kTbR;
  int n = 0;
  bool issued = false;  // A(s) already issued at this point of the order
  for (int t = 0; t <= kTbDepth - 2; ++t) {
    if (issued) n += nj;
    if (t == s) issued = true;
  }
  for (int i = 0; i <= s; ++i) {
    if (issued && i + kTbWDepth < F) n += WL;
    if (i == s) break;
    const int t = i + kTbDepth - 1;
    if (t < F) {
      if (issued) n += nj;
      if (t == s) issued = true;
    }
  }
  return n;
}

// NT: token tiles of the block that hold pairs (the block's last tiles past
// its pairs are neither loaded nor multiplied).
template <int F, int NT>
__device__ __forceinline__ void gateup_tb_body(const GateUpArgs &a, char *xs, uint32_t (*wmaxs)[64], int e,
                                               int start, int nb, int grp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int rt0 = (grp * kTbWaves + wave) * kTbR;  // row tiles rt0 .. rt0 + kTbR - 1
  constexpr int Q5 = 5 * 8 * F;  // inputs per quarter (H = 2048: 520)
  const int K = (int)a.gx.K;

  const int64_t tbytes = 64 * (int64_t)(8 * F);
  const uint8_t *gt = a.gate_p + (int64_t)e * a.stride_gu + (int64_t)rt0 * tbytes + lane * 8;
  const uint8_t *ut = a.up_p + (int64_t)e * a.stride_gu + (int64_t)rt0 * tbytes + lane * 8;
  uint2 wg[kTbWDepth][kTbR], wu[kTbWDepth][kTbR];
#define TB_WLOAD(S)                                                                                          \
  do {                                                                                                       \
    _Pragma("unroll") for (int r = 0; r < kTbR; ++r) {                                                       \
      wg[(S) % kTbWDepth][r] = *reinterpret_cast<const uint2 *>(gt + r * tbytes + (int64_t)(S) * 512);       \
      wu[(S) % kTbWDepth][r] = *reinterpret_cast<const uint2 *>(ut + r * tbytes + (int64_t)(S) * 512);       \
    }                                                                                                        \
  } while (0)

  // this wavefront's activation load instructions of a step: j = wave, wave + 8, wave + 16 (< 5 NT),
  // j = (token tile, slice m); lane (g, n) fetches 16 B of column n, quarter g
  constexpr int NJ = (5 * NT + kTbWaves - 1) / kTbWaves;
  const int nj = (wave < 5 * NT) + (wave + 8 < 5 * NT) + (wave + 16 < 5 * NT);
  const uint16_t *srow[NJ];
  int kq[NJ];
#pragma unroll
  for (int q = 0; q < NJ; ++q) {
    const int j = wave + 8 * q;
    const int tt = j / 5, m = j - tt * 5;
    const int col = min(16 * tt + n, nb - 1);
    srow[q] = a.X + (int64_t)a.sorted_token[start + col] * K;
    kq[q] = Q5 * g + 8 * m;  // input index at step 0
  }
#define TB_ALOAD(S)                                                                                          \
  do {                                                                                                       \
    char *buf_ = xs + ((S) % kTbDepth) * kTbStepBytes;                                                       \
    _Pragma("unroll") for (int q = 0; q < NJ; ++q) {                                                         \
      if (q < nj) {                                                                                          \
        const int j_ = wave + 8 * q;                                                                         \
        int k0 = kq[q] + 40 * (S);                                                                           \
        k0 = k0 < K ? k0 : K - 8;                                                                            \
        __builtin_amdgcn_global_load_lds((const void *)(srow[q] + k0),                                       \
                                         (__attribute__((address_space(3))) void *)(buf_ + j_ * 1024), 16, 0, 0); \
      }                                                                                                      \
    }                                                                                                        \
  } while (0)

#pragma unroll
  for (int s = 0; s < kTbWDepth; ++s) TB_WLOAD(s);
#pragma unroll
  for (int s = 0; s < kTbDepth - 1; ++s) TB_ALOAD(s);
  float4 sg[kTbR], su[kTbR];
#pragma unroll
  for (int r = 0; r < kTbR; ++r) {
    const int row0 = (rt0 + r) * 16 + 4 * g;
    sg[r] = *reinterpret_cast<const float4 *>(a.gate_s + (int64_t)e * a.I + row0);
    su[r] = *reinterpret_cast<const float4 *>(a.up_s + (int64_t)e * a.I + row0);
  }

  f32x4 accg[kTbR][NT], accu[kTbR][NT];
#pragma unroll
  for (int r = 0; r < kTbR; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      accg[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      accu[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
  for (int s = 0; s < F; ++s) {
    uint32_t pg[kTbR][20], pu[kTbR][20];
#pragma unroll
    for (int r = 0; r < kTbR; ++r) {
      unpack8(wg[s % kTbWDepth][r], pg[r]);
      unpack8(wu[s % kTbWDepth][r], pu[r]);
    }
    if (s + kTbWDepth < F) TB_WLOAD(s + kTbWDepth);
    // this wavefront's activation loads of step s, then everyone's; past the
    // barrier every wavefront has also finished its LDS reads of step s - 1,
    // whose buffer the next issue refills
    wait_vm(tb_after_act(s, nj, F));
    lds_barrier();
    if (s + kTbDepth - 1 < F) TB_ALOAD(s + kTbDepth - 1);
    const char *buf = xs + (s % kTbDepth) * kTbStepBytes + (g * 16 + n) * 16;
#pragma unroll
    for (int m = 0; m < 5; ++m) {
      u32x4 bx[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) bx[t] = lds16(buf + (t * 5 + m) * 1024);
#pragma unroll
      for (int r = 0; r < kTbR; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          accg[r][t] = mfma_bf16(pg[r] + 4 * m, bx[t], accg[r][t]);
          accu[r][t] = mfma_bf16(pu[r] + 4 * m, bx[t], accu[r][t]);
        }
    }
  }
#undef TB_WLOAD
#undef TB_ALOAD

  uint32_t mx[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    mx[t] = 0u;
    const int col = 16 * t + n;
#pragma unroll
    for (int r = 0; r < kTbR; ++r) {
      const int row0 = (rt0 + r) * 16 + 4 * g;
      const uint32_t m4 = store_h4(a, start + min(col, nb - 1), row0, accg[r][t], accu[r][t], sg[r], su[r],
                                   col < nb);
      mx[t] = max(mx[t], m4);
    }
    // over the four lane groups that hold the other rows of column col
    mx[t] = max(mx[t], (uint32_t)__shfl_xor((int)mx[t], 16, 64));
    mx[t] = max(mx[t], (uint32_t)__shfl_xor((int)mx[t], 32, 64));
  }
  if (g == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) wmaxs[wave][16 * t + n] = mx[t];
  }
  __syncthreads();
  if (threadIdx.x < nb) {
    uint32_t m = 0u;
#pragma unroll
    for (int w = 0; w < kTbWaves; ++w) m = max(m, wmaxs[w][threadIdx.x]);
    a.hmax[(int64_t)(start + threadIdx.x) * kTbMaxGroups + grp] = m;
  }
}

template <int F>
__global__ __launch_bounds__(64 * kTbWaves) void gateup_tb_kernel(GateUpArgs a) {
  extern __shared__ __align__(16) char xs[];  // [kTbDepth][kTbStepBytes]
  __shared__ uint32_t wmaxs[kTbWaves][64];
  const int nblk = *a.ntiles;  // here: the 64-pair blocks
  const TbItem it = tb_item(nblk, a.I / kTbRows);
  if (it.blk >= nblk) return;
  const int4 td = reinterpret_cast<const int4 *>(a.tiles)[it.blk];
  const int e = td.x, start = td.y;
  const int nb = td.z;  // pairs of this block (1..64)
  switch ((nb + 15) >> 4) {
    case 1: gateup_tb_body<F, 1>(a, xs, wmaxs, e, start, nb, it.grp); break;
    case 2: gateup_tb_body<F, 2>(a, xs, wmaxs, e, start, nb, it.grp); break;
    case 3: gateup_tb_body<F, 3>(a, xs, wmaxs, e, start, nb, it.grp); break;
    default: gateup_tb_body<F, 4>(a, xs, wmaxs, e, start, nb, it.grp); break;
  }
}

// ----------------------------------------------------------------- down
struct DownArgs {
  const uint8_t *down_p;
  int64_t stride_d;
  const float *down_s;
  const float *hf;        // [pairs][I] fp32 h in grouped order
  const uint32_t *hmax;   // token-blocked path: [pairs][kTbMaxGroups] largest |h| per row group
  int hgroups;            // row groups in hmax
  const int32_t *tiles, *ntiles;
  float *O;  // [pairs][H]
  int H, I, slots;
  Geom gd;       // operand geometry of the down projection (K = I)
  int stream_w;  // few pairs per expert: each weight tile is read once, non-temporally
};

// Workgroup = 4 wavefronts x R 16-row tiles each (64 R output rows); two fp16
// passes (the hi and lo parts of the scaled h) per operand slice, each slice
// read from LDS once per wavefront for its R row tiles.
template <int F, int RT, int R>
__device__ inline void down_work(const DownArgs &a, char *smem, int tile, int ry) {
  const int4 td = reinterpret_cast<const int4 *>(a.tiles)[tile];
  const int e = td.x, start = td.y, cnt = td.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int M = 5 * F + tail_mfmas(RT);
  const int rtb = ry * 4 * R + wave;  // row tiles rtb + 4 r
  const int rs = lds_row_bytes(a.slots);
  char *xb[2] = {smem, smem + 17 * rs};  // [2][17][rs]
  const int g = lane >> 4;

  const int64_t tbytes = 64 * (int64_t)(8 * F + RT);
  uint2 dd[R][F];
  uint32_t ddw[R], dsh[R];
  float4 sd[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint8_t *dt = a.down_p + (int64_t)e * a.stride_d + (int64_t)(rtb + 4 * r) * tbytes;
#pragma unroll
    for (int s = 0; s < F; ++s)
      dd[r][s] = a.stream_w ? ldw8(dt + (int64_t)s * 512 + lane * 8)
                            : *reinterpret_cast<const uint2 *>(dt + (int64_t)s * 512 + lane * 8);
    ddw[r] = dsh[r] = 0;
    if constexpr (RT > 0) load_tail<RT>(dt, F, lane, ddw[r], dsh[r]);
    sd[r] = *reinterpret_cast<const float4 *>(a.down_s + (int64_t)e * a.H + (rtb + 4 * r) * 16 + 4 * g);
  }

  __shared__ int sig[16];
  stage_h_parts<4, 4, M>(a.hf + (int64_t)start * a.I, cnt, a.I, 5 * a.gd.Q, xb[0], xb[1], rs, sig);
#pragma unroll
  for (int q = 0; q < 2; ++q) zero_row(xb[q] + 16 * rs, a.slots, threadIdx.x, 256);
  __syncthreads();

  const int n = lane & 15;
  const int boff = (n < cnt ? n : 16) * rs + g * M * 16;
  f32x4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < F; ++s) {
    u32x4 bx[5][2];
#pragma unroll
    for (int m = 0; m < 5; ++m)
#pragma unroll
      for (int q = 0; q < 2; ++q) bx[m][q] = lds16(xb[q] + boff + (5 * s + m) * 16);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t pw[20];
      unpack8(dd[r][s], pw);
#pragma unroll
      for (int m = 0; m < 5; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[r] = mfma_f16(pw + 4 * m, bx[m][q], acc[r]);
    }
  }
  if constexpr (RT > 0) {
    u32x4 bx[tail_mfmas(RT)][2];
#pragma unroll
    for (int m = 0; m < tail_mfmas(RT); ++m)
#pragma unroll
      for (int q = 0; q < 2; ++q) bx[m][q] = lds16(xb[q] + boff + (5 * F + m) * 16);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t pw[16];
      unpack_tail<RT>(ddw[r], dsh[r], pw);
#pragma unroll
      for (int m = 0; m < tail_mfmas(RT); ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc[r] = mfma_f16(pw + 4 * m, bx[m][q], acc[r]);
    }
  }
  if (n >= cnt) return;
  const int64_t p = start + n;
  const int us = -1 - sig[n];  // the trits entered as 2t, h as 2^sig h
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row0 = (rtb + 4 * r) * 16 + 4 * g;
    float4 o;
    o.x = ldexpf(acc[r][0], us) * sd[r].x;
    o.y = ldexpf(acc[r][1], us) * sd[r].y;
    o.z = ldexpf(acc[r][2], us) * sd[r].z;
    o.w = ldexpf(acc[r][3], us) * sd[r].w;
    *reinterpret_cast<float4 *>(a.O + p * a.H + row0) = o;
  }
}

// A fixed grid walking the (work tile, 64 R-row group) items.
template <int F, int RT, int R>
__global__ __launch_bounds__(256) void down_kernel(DownArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int groups = a.H / 64 / R;
  const int nitems = *a.ntiles * groups;
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int tile = item / groups;
    down_work<F, RT, R>(a, smem, tile, item - tile * groups);
    __syncthreads();  // the staged h parts are reused by the next item
  }
}

// ------------------------------------------------ down, token-blocked
// Many pairs per expert (prefill): a workgroup takes one of the gate/up
// blocks (up to 64 pairs of one expert) and H / kDtbGroups output rows. The
// block's h rows are staged once as their scaled fp16 parts (two planes of 64
// rows, 138 KB of LDS); each wavefront then walks its row tiles kDtbR at a
// time: the weights of a K step are decoded once and feed 4 token tiles x 2
// parts x kDtbR row tiles, and each operand slice read from LDS feeds kDtbR
// products. Columns past the block read its last pair and are not stored. The next row tiles' weights are in
// flight while the current ones are multiplied (the first ones while h is
// staged).
constexpr int kDtbWaves = 8, kDtbR = 4, kDtbGroups = 4;
// workgroups of the persistent token-blocked down: one per CU (its 138 KB of
// LDS leave room for one), a multiple of 8
static unsigned dtb_grid() {
  // read once (thread-safe static initialization); any multiple of 8 is
  // correct, the CU count only balances the runs
  static const unsigned n = []() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    return (unsigned)((cus + 7) / 8 * 8);
  }();
  return n;
}

template <int F, int RT>
struct DtbWeights {
  uint2 d[kDtbR][F];
  uint32_t dw[kDtbR], sh[kDtbR];
};

template <int F, int RT>
__device__ __forceinline__ void dtb_load(const DownArgs &a, int e, int rt, int lane, DtbWeights<F, RT> &w) {
  const int64_t tbytes = 64 * (int64_t)(8 * F + RT);
#pragma unroll
  for (int r = 0; r < kDtbR; ++r) {
    const uint8_t *dt = a.down_p + (int64_t)e * a.stride_d + (int64_t)(rt + r) * tbytes;
#pragma unroll
    for (int s = 0; s < F; ++s) w.d[r][s] = *reinterpret_cast<const uint2 *>(dt + (int64_t)s * 512 + lane * 8);
    w.dw[r] = w.sh[r] = 0;
    if constexpr (RT > 0) load_tail<RT>(dt, F, lane, w.dw[r], w.sh[r]);
  }
}

// One operand slice: the hi parts of the 4 token tiles into every row tile's
// accumulator, then the lo parts (so no two consecutive products share an
// accumulator). All four token tiles run (straight-line code schedules the
// LDS reads ahead of the products); columns past the block read its last pair.
template <int NT, int NW>
__device__ __forceinline__ void dtb_slice(const uint32_t (*pw)[NW], int w0, const char *base, const int bq[NT],
                                          int plane, int off, f32x4 (*acc)[NT]) {
  u32x4 b[2][NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    b[0][t] = lds16(base + bq[t] + off);
    b[1][t] = lds16(base + bq[t] + plane + off);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < kDtbR; ++r) acc[r][t] = mfma_f16(pw[r] + w0, b[q][t], acc[r][t]);
}

// Persistent walk: gridDim.x workgroups (a multiple of 8, one per CU) take
// contiguous runs of the (block, row group) items, kDtbGroups items per block
// in order, the runs of XCD x (workgroups x, x + 8, ...) next to each other.
// A workgroup stages a block's h once for all of that block's items it runs
// (a block change waits for every wavefront, then restages), and issues the
// next item's weights during the current item's last K step. All four token
// tiles are multiplied (a form per live-tile count would need more than the
// 256 registers two wavefronts per SIMD leave each); columns past the block's
// pairs read its last pair and are not stored.
template <int F, int RT>
__global__ __launch_bounds__(64 * kDtbWaves) void down_tb_kernel(DownArgs a) {
  extern __shared__ __align__(16) char smem[];  // [2][64][rs]: the hi and lo planes
  __shared__ int sig[64];
  constexpr int NT = 4, G = kDtbGroups;
  constexpr int M = 5 * F + tail_mfmas(RT);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int rs = lds_row_bytes(a.slots);
  const int plane = 64 * rs;
  const int nitems = *a.ntiles * G;  // here: the 64-pair blocks
  const int nwg = (int)gridDim.x;
  const int run = (int)(blockIdx.x & 7) * (nwg >> 3) + (int)(blockIdx.x >> 3);
  const int per = (nitems + nwg - 1) / nwg;
  const int i0 = min(run * per, nitems), i1 = min(i0 + per, nitems);
  if (i0 >= i1) return;
  const int rows_g = a.H / 16 / G;  // row tiles of an item: kDtbR per wavefront
  const int4 *tiles = reinterpret_cast<const int4 *>(a.tiles);

  int blk = -1, e = 0, start = 0, nb = 1;
  DtbWeights<F, RT> cur;
#pragma unroll 1
  for (int item = i0; item < i1; ++item) {
    if (item / G != blk) {
      // a new block: every wavefront has finished reading the last one's h and
      // sig; its h is staged (the run's first item: its weights behind h; the
      // later items' weights are already in flight)
      if (blk >= 0) __syncthreads();
      blk = item / G;
      const int4 td = tiles[blk];
      e = td.x;
      start = td.y;
      nb = td.z;  // 1..64 pairs
      stage_h_known<64 * kDtbWaves, M>(a.hf + (int64_t)start * a.I, a.hmax + (int64_t)start * kTbMaxGroups,
                                       a.hgroups, nb, a.I, 5 * a.gd.Q, smem, smem + plane, rs, sig, [&]() {
                                         if (item == i0) dtb_load<F, RT>(a, e, (i0 % G) * rows_g + wave * kDtbR, lane, cur);
                                       });
      __syncthreads();
    }
    const int rt0 = (item % G) * rows_g + wave * kDtbR;  // this wavefront's kDtbR row tiles
    // the next item of the run (the last one again after the last): its block's tiles
    const int nxt = min(item + 1, i1 - 1);
    const int4 ntd = tiles[nxt / G];
    int bq[NT];  // LDS offsets of the four token tiles' operand rows
#pragma unroll
    for (int t = 0; t < NT; ++t) bq[t] = min(16 * t + n, nb - 1) * rs + g * M * 16;
    f32x4 acc[kDtbR][NT];
#pragma unroll
    for (int r = 0; r < kDtbR; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the row scales, needed only by the epilogue
    float4 sd[kDtbR];
#pragma unroll
    for (int r = 0; r < kDtbR; ++r)
      sd[r] = *reinterpret_cast<const float4 *>(a.down_s + (int64_t)e * a.H + (rt0 + r) * 16 + 4 * g);
    // after the last step is decoded the weight registers are free for the
    // next item's row tiles, which land while that step's products run
    if constexpr (RT > 0) {
      uint32_t pw[kDtbR][16];
#pragma unroll
      for (int r = 0; r < kDtbR; ++r) unpack_tail<RT>(cur.dw[r], cur.sh[r], pw[r]);
#pragma unroll
      for (int m = 0; m < tail_mfmas(RT); ++m) {
        dtb_slice<NT>(pw, 4 * m, smem, bq, plane, (5 * F + m) * 16, acc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int s = 0; s < F; ++s) {
      uint32_t pw[kDtbR][20];
#pragma unroll
      for (int r = 0; r < kDtbR; ++r) unpack8(cur.d[r][s], pw[r]);
      if (s == F - 1) dtb_load<F, RT>(a, ntd.x, (nxt % G) * rows_g + wave * kDtbR, lane, cur);
#pragma unroll
      for (int m = 0; m < 5; ++m) {
        dtb_slice<NT>(pw, 4 * m, smem, bq, plane, (5 * s + m) * 16, acc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int col = 16 * t + n;
      if (col >= nb) continue;
      const int us = -1 - sig[col];  // the trits entered as 2t, h as 2^sig h
      float *op = a.O + (int64_t)(start + col) * a.H;
#pragma unroll
      for (int r = 0; r < kDtbR; ++r) {
        const int row0 = (rt0 + r) * 16 + 4 * g;
        float4 o;
        o.x = ldexpf(acc[r][t][0], us) * sd[r].x;
        o.y = ldexpf(acc[r][t][1], us) * sd[r].y;
        o.z = ldexpf(acc[r][t][2], us) * sd[r].z;
        o.w = ldexpf(acc[r][t][3], us) * sd[r].w;
        *reinterpret_cast<float4 *>(op + row0) = o;
      }
    }
  }
}

// ------------------------------------------------- down + combine (decode)
struct DownCombineArgs {
  const uint8_t *down_p;
  int64_t stride_d;
  const float *down_s;
  const float *hf;  // [pairs][I] fp32 h in grouped order
  int slots, I;
  const int32_t *tiles, *ntiles, *sorted_token;
  const float *pair_w;  // [pairs] routing weight of each grouped pair
  int P, T, H, max_tiles;
  Geom gd;  // operand geometry of the down projection (K = I)
  float *Y;                   // [T][H] or null
  const uint16_t *resid_in;   // [T][H] bf16 or null
  uint16_t *resid_out;        // [T][H] bf16 or null (may alias resid_in)
};

constexpr int kDcWaves = 8;

// Decode path with few pairs (T*k <= 32): workgroup = one 16-row block of the
// H outputs for all work tiles. The two fp16 parts of the scaled h of every
// pair are staged in LDS (the first tile's weights in flight meanwhile);
// wavefront w then takes
// tiles w, w + 8, ... in order and adds pair_w * o (o = sd * (Td h)) into its
// own LDS accumulator of the pair's token; the accumulators are summed in fixed
// order, then Y and/or the residual bf16(x + y) are written. MFMA columns past
// the tile's pairs repeat its last pair and are discarded.
template <int F, int RT>
__global__ __launch_bounds__(64 * kDcWaves) void down_combine_kernel(DownCombineArgs a) {
  extern __shared__ __align__(16) char hps[];  // [2][P][slots] fp16
  __shared__ float yacc[kDcWaves][kDecodeMaxT][16];
  __shared__ int32_t s_tok[kDcMaxPairs];
  __shared__ float s_pw[kDcMaxPairs];
  __shared__ int s_sig[kDcMaxPairs];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rt = blockIdx.x;
  constexpr int M = 5 * F + tail_mfmas(RT);
  const int n = lane & 15, g = lane >> 4;
  const int64_t tbytes = 64 * (int64_t)(8 * F + RT);
  const int nt = *a.ntiles;
  // first tile (before nt is known), then each pair's token and weight: all
  // issued unconditionally (clamped indices), so they share one round trip
  const int4 td0 = reinterpret_cast<const int4 *>(a.tiles)[min(wave, a.max_tiles - 1)];
  const int pi = min((int)threadIdx.x, a.P - 1);
  const int32_t tok_i = a.sorted_token[pi];
  const float pw_i = a.pair_w[pi];
  // the first tile's weights in flight while h is staged
  uint2 dd0[F];
  uint32_t ddw0 = 0, dsh0 = 0;
  float4 sd0 = make_float4(0.f, 0.f, 0.f, 0.f);
  if (wave < nt) {
    const uint8_t *dt = a.down_p + (int64_t)td0.x * a.stride_d + (int64_t)rt * tbytes;
#pragma unroll
    for (int s = 0; s < F; ++s) dd0[s] = ldw8(dt + (int64_t)s * 512 + lane * 8);
    if constexpr (RT > 0) load_tail<RT>(dt, F, lane, ddw0, dsh0);
    sd0 = *reinterpret_cast<const float4 *>(a.down_s + (int64_t)td0.x * a.H + rt * 16 + 4 * g);
  }
  const int plane = a.P * a.slots * 2;
  stage_h_parts<kDcWaves, kDcMaxPairs / kDcWaves, M>(a.hf, a.P, a.I, 5 * a.gd.Q, hps, hps + plane, a.slots * 2,
                                                     s_sig);
  if ((int)threadIdx.x < a.P) {
    s_tok[threadIdx.x] = tok_i;
    s_pw[threadIdx.x] = pw_i;
  }
  for (int i = lane; i < kDecodeMaxT * 16; i += 64) (&yacc[wave][0][0])[i] = 0.f;
  lds_barrier();  // the first tile's weights may still be in flight
  for (int tile = wave; tile < nt; tile += kDcWaves) {
    const bool first = tile == wave;
    const int4 td = first ? td0 : reinterpret_cast<const int4 *>(a.tiles)[tile];
    const int e = td.x, start = td.y, cnt = td.z;
    uint2 dd[F];
    uint32_t ddw = ddw0, dsh = dsh0;
    float4 sd = sd0;
    if (first) {
#pragma unroll
      for (int s = 0; s < F; ++s) dd[s] = dd0[s];
    } else {
      const uint8_t *dt = a.down_p + (int64_t)e * a.stride_d + (int64_t)rt * tbytes;
#pragma unroll
      for (int s = 0; s < F; ++s) dd[s] = ldw8(dt + (int64_t)s * 512 + lane * 8);
      if constexpr (RT > 0) load_tail<RT>(dt, F, lane, ddw, dsh);
      sd = *reinterpret_cast<const float4 *>(a.down_s + (int64_t)e * a.H + rt * 16 + 4 * g);
    }
    const bool live = n < cnt;
    const int p = start + (live ? n : cnt - 1);
    const char *hb = hps + p * a.slots * 2 + g * 16 * M;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < F; ++s) {
      uint32_t pw[20];
      unpack8(dd[s], pw);
#pragma unroll
      for (int m = 0; m < 5; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc = mfma_f16(pw + 4 * m, lds16(hb + q * plane + 16 * (5 * s + m)), acc);
    }
    if constexpr (RT > 0) {
      uint32_t pw[16];
      unpack_tail<RT>(ddw, dsh, pw);
#pragma unroll
      for (int m = 0; m < tail_mfmas(RT); ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) acc = mfma_f16(pw + 4 * m, lds16(hb + q * plane + 16 * (5 * F + m)), acc);
    }
    if (live) {
      const int tok = s_tok[p];
      const float wt = s_pw[p];
      const int us = -1 - s_sig[p];  // the trits entered as 2t, h as 2^sig h
      const float sdv[4] = {sd.x, sd.y, sd.z, sd.w};
#pragma unroll
      for (int v = 0; v < 4; ++v)
        yacc[wave][tok][4 * g + v] = fmaf(wt, ldexpf(acc[v], us) * sdv[v], yacc[wave][tok][4 * g + v]);
    }
  }
  __syncthreads();
  const int i = threadIdx.x;
  if (i < a.T * 16) {
    const int t = i >> 4, r = i & 15;
    float y = yacc[0][t][r];
#pragma unroll
    for (int w = 1; w < kDcWaves; ++w) y += yacc[w][t][r];
    const int64_t o = (int64_t)t * a.H + rt * 16 + r;
    if (a.Y) a.Y[o] = y;
    if (a.resid_out) a.resid_out[o] = f32_to_bf16_rne(__uint_as_float((uint32_t)a.resid_in[o] << 16) + y);
  }
}

// ---------------------------------------------------------- ternary linear
struct LinearArgs {
  const uint8_t *pt;
  const float *s;
  const uint16_t *X;  // [T][ldx] bf16, natural order
  float *Y;
  int64_t T, N, ldx, ldy;
  Geom g;
  bool contig;
  bool rows_x;  // grid x walks the row-tile groups (one token tile), else the token tiles
  int zrow;     // staged rows per token tile (min(16, T)); this LDS row holds zeros
};

// blockIdx.x = 16-token tile, blockIdx.y = group of 4/KS row tiles (swapped
// when rows_x: one token tile and up to 2^31 row groups). F < 0: generic K
// (runtime steps, one step in flight). LDS holds zrow + 1 rows.
template <int F, int RT, int KS>
__global__ __launch_bounds__(256) void linear_kernel(LinearArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int RTB = 4 / KS;
  const int64_t t0 = (int64_t)(a.rows_x ? blockIdx.y : blockIdx.x) * 16;
  const int cnt = (int)min<int64_t>(16, a.T - t0);
  const int nrt = (int)((a.N + 15) / 16);
  const int rt = (int)(a.rows_x ? blockIdx.x : blockIdx.y) * RTB + wave / KS;
  const int kp = wave % KS;
  const bool active = rt < nrt;
  const int rs = lds_row_bytes(a.g.slots);
  const int Fr = F >= 0 ? F : a.g.F;
  const int Rr = F >= 0 ? RT : a.g.r;
  const int M = 5 * Fr + (Rr == 0 ? 0 : (5 * (Rr / 2) + 3) / 4);
  const int64_t tbytes = 64 * (int64_t)(8 * Fr + Rr);
  const uint8_t *wt = a.pt + (int64_t)(active ? rt : 0) * tbytes;
  char *xs = smem;
  const int s0 = kp * Fr / KS, s1 = (kp + 1) * Fr / KS;
  const bool tail_here = Rr > 0 && kp == KS - 1;
  // fixed K: this wavefront's weights first, in flight while the activations are staged
  constexpr int SMAXF = F >= 0 ? (F + KS - 1) / KS : 1;
  uint2 dpre[SMAXF > 0 ? SMAXF : 1];
  uint32_t dwpre = 0, shpre = 0;
  if constexpr (F >= 0) {
    if (active) {
#pragma unroll
      for (int i = 0; i < SMAXF; ++i)
        if (s0 + i < s1) dpre[i] = *reinterpret_cast<const uint2 *>(wt + (int64_t)(s0 + i) * 512 + lane * 8);
      if (tail_here) load_tail<RT>(wt, F, lane, dwpre, shpre);
    }
  }

  if (a.contig) {
    const int vec = a.g.slots / 8, kv = (int)(a.g.K / 8);
    copy16<256>(
        cnt * vec,
        [&](int i) {
          const int n = i / vec, c = i - n * vec;
          return c < kv ? reinterpret_cast<const uint4 *>(a.X + (t0 + n) * a.ldx)[c] : make_uint4(0, 0, 0, 0);
        },
        [&](int i) {
          const int n = i / vec, c = i - n * vec;
          return reinterpret_cast<uint4 *>(xs + n * rs + c * 16);
        });
  } else {
    for (int n = 0; n < cnt; ++n) stage_row(xs + n * rs, a.X + (t0 + n) * a.ldx, a.g, threadIdx.x, 256);
  }
  zero_row(xs + a.zrow * rs, a.g.slots, threadIdx.x, 256);
  __syncthreads();

  const int n = lane & 15, g = lane >> 4;
  const char *bp = xs + (n < cnt ? n : a.zrow) * rs + g * M * 16;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    if constexpr (F >= 0) {
      constexpr int SMAX = SMAXF;
      const uint2 *d = dpre;
      const uint32_t dw = dwpre, sh = shpre;
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
    float *red = reinterpret_cast<float *>(smem + (a.zrow + 1) * rs);  // [4][64][4]
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

// ------------------------------------------- ternary linear, streamed
// Few tokens over very many rows (K = 2048): each workgroup stages the tokens
// once, then every wavefront walks its own row tiles (wavefront g of G takes
// tiles g, g + G, ...), the next tile's weights and row scales in flight while
// the current one is decoded and multiplied. Nothing synchronizes the
// wavefronts after the staging, so loads from many tiles per CU overlap.
constexpr int kStreamWgs = 1024;  // four workgroups of four wavefronts per CU (about 110 VGPRs each)

struct StreamW {
  uint2 d[13];
  float4 sc;
};

__device__ __forceinline__ void stream_issue(const LinearArgs &a, int rt, int nrt, int lane, StreamW &w) {
  const bool live = rt < nrt;  // otherwise every lane reads the first bytes (counts stay path-independent)
  const int64_t base = live ? (int64_t)rt * (64 * 8 * 13) + lane * 8 : 0;
  const int64_t step = live ? 512 : 0;
#pragma unroll
  for (int s = 0; s < 13; ++s) w.d[s] = ldw8(a.pt + base + s * step);
  const int64_t row0 = (int64_t)rt * 16 + 4 * (lane >> 4);
  w.sc = live && row0 + 3 < a.N ? *reinterpret_cast<const float4 *>(a.s + row0) : make_float4(0.f, 0.f, 0.f, 0.f);
  if (live && row0 + 3 >= a.N) {  // the last, partial row tile
    w.sc.x = row0 < a.N ? a.s[row0] : 0.f;
    w.sc.y = row0 + 1 < a.N ? a.s[row0 + 1] : 0.f;
    w.sc.z = row0 + 2 < a.N ? a.s[row0 + 2] : 0.f;
  }
}

__global__ __launch_bounds__(256) void linear_stream_kernel(LinearArgs a) {
  extern __shared__ __align__(16) char smem[];  // [zrow + 1][rs]
  constexpr int M = 65;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cnt = (int)a.T;  // <= 16, one token tile
  const int nrt = (int)((a.N + 15) / 16);
  const int rs = lds_row_bytes(a.g.slots);
  const int G = gridDim.x * 4;
  int rt = blockIdx.x * 4 + wave;
  StreamW cur, nxt;
  stream_issue(a, rt, nrt, lane, cur);
  {
    const int vec = a.g.slots / 8, kv = 256;  // natural operand order, K = 2048
    copy16<256>(
        cnt * vec,
        [&](int i) {
          const int n = i / vec, c = i - n * vec;
          return c < kv ? reinterpret_cast<const uint4 *>(a.X + n * a.ldx)[c] : make_uint4(0, 0, 0, 0);
        },
        [&](int i) {
          const int n = i / vec, c = i - n * vec;
          return reinterpret_cast<uint4 *>(smem + n * rs + c * 16);
        });
    zero_row(smem + a.zrow * rs, a.g.slots, threadIdx.x, 256);
  }
  __syncthreads();
  const int n = lane & 15, g = lane >> 4;
  int boff = (n < cnt ? n : a.zrow) * rs + g * M * 16;
#pragma nounroll
  for (; rt < nrt; rt += G) {
    // the activation slices are re-read from LDS every tile (an opaque offset
    // keeps the compiler from hoisting all 65 of them into 260 registers,
    // which would leave one wavefront per SIMD)
    asm volatile("" : "+v"(boff));
    const char *bp = smem + boff;
    stream_issue(a, rt + G, nrt, lane, nxt);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 13; ++s) {
      uint32_t pw[20];
      unpack8(cur.d[s], pw);
#pragma unroll
      for (int m = 0; m < 5; ++m) acc = mfma_bf16(pw + 4 * m, lds16(bp + (5 * s + m) * 16), acc);
    }
    if (n < cnt) {
      const int64_t row0 = (int64_t)rt * 16 + 4 * g;
      float *y = a.Y + n * a.ldy;
      const float sv[4] = {cur.sc.x, cur.sc.y, cur.sc.z, cur.sc.w};
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (row0 + v < a.N) y[row0 + v] = (acc[v] * 0.5f) * sv[v];
    }
    cur = nxt;
  }
}

// ------------------------------------------- ternary linear, fp32 input
// Y = s (.) (T x) with fp32 x: while staging, each input is split exactly into
// three bf16 parts (hi + mid + lo, exact: each rounding keeps the next 8 of
// the 24 significant bits), and every
// decoded weight slice multiplies all three (fp32 accumulation). Optional
// residual: resid_out = bf16(fp32(resid_in) + y). K = 2048 only (natural
// operand order); eight tokens per workgroup (three planes of staged rows).
struct Linear3Args {
  const uint8_t *pt;
  const float *s;
  const float *X;  // [T][K] fp32
  float *Y;        // [T][N] or null
  const uint16_t *resid_in;
  uint16_t *resid_out;  // [T][N] bf16 or null
  int64_t T, N;
  Geom g;
};
constexpr int kL3Tok = 8;

template <int KS>
__global__ __launch_bounds__(256) void linear3_kernel(Linear3Args a) {
  extern __shared__ __align__(16) char smem[];
  constexpr int F = 13, TT = kL3Tok, RTB = 4 / KS, M = 5 * F;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * TT;
  const int cnt = (int)min<int64_t>(TT, a.T - t0);
  const int nrt = (int)((a.N + 15) / 16);
  const int rt = blockIdx.y * RTB + wave / KS;
  const int kp = wave % KS;
  const bool active = rt < nrt;
  const int rs = lds_row_bytes(a.g.slots);
  const int plane = (TT + 1) * rs;  // [3][TT + 1][rs]; row TT of each plane is zero
  const uint8_t *wt = a.pt + (int64_t)(active ? rt : 0) * (64 * 8 * F);
  // this wavefront's weights first: in flight while the activations are staged
  constexpr int SMAX = (F + KS - 1) / KS;
  const int s0 = kp * F / KS, s1 = (kp + 1) * F / KS;
  uint2 d[SMAX];
#pragma unroll
  for (int i = 0; i < SMAX; ++i)
    if (active && s0 + i < s1) d[i] = ldw8(wt + (int64_t)(s0 + i) * 512 + lane * 8);
  const int vec = a.g.slots / 8, kv = (int)(a.g.K / 8);
  for (int i = threadIdx.x; i < cnt * vec; i += 256) {
    const int n = i / vec, c = i - n * vec;
    uint32_t w3[3][4] = {};
    if (c < kv) {
      const float4 *src = reinterpret_cast<const float4 *>(a.X + (t0 + n) * a.g.K) + 2 * c;
      const float4 f0 = src[0], f1 = src[1];
      const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t b0 = f32_to_bf16_rne(f[e]);
        const float r1 = f[e] - __uint_as_float(b0 << 16);
        const uint32_t b1 = f32_to_bf16_rne(r1);
        const uint32_t b2 = f32_to_bf16_rne(r1 - __uint_as_float(b1 << 16));
        const int sh = 16 * (e & 1);
        w3[0][e >> 1] |= b0 << sh;
        w3[1][e >> 1] |= b1 << sh;
        w3[2][e >> 1] |= b2 << sh;
      }
    }
#pragma unroll
    for (int q = 0; q < 3; ++q)
      *reinterpret_cast<uint4 *>(smem + q * plane + n * rs + c * 16) = make_uint4(w3[q][0], w3[q][1], w3[q][2], w3[q][3]);
  }
#pragma unroll
  for (int q = 0; q < 3; ++q) zero_row(smem + q * plane + TT * rs, a.g.slots, threadIdx.x, 256);
  __syncthreads();

  const int n = lane & 15, g = lane >> 4;
  const char *bp = smem + (n < cnt ? n : TT) * rs + g * M * 16;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (active) {
#pragma unroll
    for (int i = 0; i < SMAX; ++i) {
      const int st = s0 + i;
      if (st < s1) {
        uint32_t pw[20];
        unpack8(d[i], pw);
#pragma unroll
        for (int m = 0; m < 5; ++m)
#pragma unroll
          for (int q = 0; q < 3; ++q) acc = mfma_bf16(pw + 4 * m, lds16(bp + q * plane + (5 * st + m) * 16), acc);
      }
    }
  }
  if constexpr (KS > 1) {
    float *red = reinterpret_cast<float *>(smem + 3 * plane);  // [4][64][4]
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
  const int64_t row0 = (int64_t)rt * 16 + 4 * g, t = t0 + n;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t row = row0 + v;
    if (row >= a.N) continue;
    const float y = (acc[v] * 0.5f) * a.s[row];
    if (a.Y) a.Y[t * a.N + row] = y;
    if (a.resid_out)
      a.resid_out[t * a.N + row] = f32_to_bf16_rne(__uint_as_float((uint32_t)a.resid_in[t * a.N + row] << 16) + y);
  }
}

// ------------------------------------------------------------------ combine
// grid (T, H / (512 C)), 128 threads x C float4 columns each (128 apart, so
// every load instruction of the workgroup is contiguous); fixed slot order
// j = 0..k-1 (slots with pos < 0 are skipped). The slots go 8 at a time with
// all 8 C output rows in flight before the first product: no load sits under a
// branch (an invalid slot reads row 0 and is dropped by a select, so nothing it
// holds can reach the sum), which would make each product wait for its own
// load. NT: the expert outputs are far larger than the caches and read once,
// non-temporally. C = 2 for large batches (twice the loads in flight per
// thread); C = 1 keeps enough workgroups for a few tokens.
template <bool NT, int C>
__global__ __launch_bounds__(128) void combine_kernel(const float *O, const float *w, const int32_t *pos, int k,
                                                       int H, float *Y, const uint16_t *resid_in,
                                                       uint16_t *resid_out) {
  constexpr int B = 8;
  const int64_t t = blockIdx.x;
  const int cb = blockIdx.y * 128 * C + threadIdx.x;  // float4 column of q = 0
  uint2 xi[C];  // the residual input, fetched with the first slots
#pragma unroll
  for (int q = 0; q < C; ++q) {
    const int c = cb + 128 * q;
    xi[q] = make_uint2(0u, 0u);
    if (resid_out && c * 4 < H) xi[q] = reinterpret_cast<const uint2 *>(resid_in + t * H)[c];
  }
  float4 acc[C];
#pragma unroll
  for (int q = 0; q < C; ++q) acc[q] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < k; j0 += B) {
    int pj[B];
    float wj[B];
    f32x4 o[B][C];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int j = min(j0 + u, k - 1);
      pj[u] = pos[t * k + j];
      wj[u] = w[t * k + j];
    }
#pragma unroll
    for (int u = 0; u < B; ++u)
#pragma unroll
      for (int q = 0; q < C; ++q) {
        // columns past H read the row's last column (dropped below)
        const int c = min(cb + 128 * q, H / 4 - 1);
        const f32x4 *src = reinterpret_cast<const f32x4 *>(O + (int64_t)max(pj[u], 0) * H) + c;
        if constexpr (NT) o[u][q] = __builtin_nontemporal_load(src);
        else o[u][q] = *src;
      }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const bool use = j0 + u < k && pj[u] >= 0;
#pragma unroll
      for (int q = 0; q < C; ++q) {
        acc[q].x = use ? fmaf(wj[u], o[u][q][0], acc[q].x) : acc[q].x;
        acc[q].y = use ? fmaf(wj[u], o[u][q][1], acc[q].y) : acc[q].y;
        acc[q].z = use ? fmaf(wj[u], o[u][q][2], acc[q].z) : acc[q].z;
        acc[q].w = use ? fmaf(wj[u], o[u][q][3], acc[q].w) : acc[q].w;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < C; ++q) {
    const int c = cb + 128 * q;
    if (c * 4 >= H) continue;
    if (Y) reinterpret_cast<float4 *>(Y + t * H)[c] = acc[q];
    if (resid_out) {
      const float x0 = __uint_as_float(xi[q].x << 16), x1 = __uint_as_float(xi[q].x & 0xFFFF0000u);
      const float x2 = __uint_as_float(xi[q].y << 16), x3 = __uint_as_float(xi[q].y & 0xFFFF0000u);
      uint2 r;
      r.x = (uint32_t)f32_to_bf16_rne(x0 + acc[q].x) | ((uint32_t)f32_to_bf16_rne(x1 + acc[q].y) << 16);
      r.y = (uint32_t)f32_to_bf16_rne(x2 + acc[q].z) | ((uint32_t)f32_to_bf16_rne(x3 + acc[q].w) << 16);
      reinterpret_cast<uint2 *>(resid_out + t * H)[c] = r;
    }
  }
}

// ----------------------------------------------------------------- host side
int64_t ffn_max_tiles(int64_t pairs, int64_t E) { return cdiv(pairs, 16) + (pairs < E ? pairs : E); }
static int64_t ffn_max_blocks(int64_t pairs, int64_t E) { return cdiv(pairs, 64) + (pairs < E ? pairs : E); }

size_t ffn_ws_bytes(int64_t T, int k, int64_t E, int64_t H, int64_t I) {
  (void)H;
  const int64_t P = T * k;
  size_t o = 0;
  o = align_up(o + ffn_max_tiles(P, E) * 16, 256);
  o = align_up(o + 16, 256);
  o = align_up(o + (size_t)P * I * 4, 256);
  o = align_up(o + (size_t)P * 4, 256);
  o = align_up(o + ffn_max_blocks(P, E) * 16, 256);
  o = align_up(o + 16, 256);
  o = align_up(o + (size_t)P * kTbMaxGroups * 4, 256);
  return o;
}

FfnWs ffn_ws_carve(void *ws, int64_t T, int k, int64_t E, int64_t H, int64_t I) {
  (void)H;
  const int64_t P = T * k;
  char *b = (char *)ws;
  FfnWs f;
  size_t o = 0;
  f.tiles = (int32_t *)(b + o);
  o = align_up(o + ffn_max_tiles(P, E) * 16, 256);
  f.ntiles = (int32_t *)(b + o);
  o = align_up(o + 16, 256);
  f.hf = (float *)(b + o);
  o = align_up(o + (size_t)P * I * 4, 256);
  f.pw = (float *)(b + o);
  o = align_up(o + (size_t)P * 4, 256);
  f.blocks = (int32_t *)(b + o);
  o = align_up(o + ffn_max_blocks(P, E) * 16, 256);
  f.nblocks = (int32_t *)(b + o);
  o = align_up(o + 16, 256);
  f.hmax = (uint32_t *)(b + o);
  return f;
}

template <int F, int RT, int KS, int RNPL, int R = 1, int NW = 4>
static int run_gateup(hipStream_t st, const GateUpArgs &a, int64_t max_tiles, int I, bool walk = true) {
  const int rs = lds_row_bytes(a.gx.slots);
  size_t lds = (size_t)17 * rs + (KS > 1 ? 4 * 64 * 8 * 4 : 0);
  const int64_t groups = I / 16 / (NW / KS) / R;
  dim3 grid((unsigned)max_tiles, (unsigned)groups);
  if (RNPL == 0) grid = dim3(walk_grid(max_tiles * groups, walk), 1);
  int rc = allow_lds<gateup_kernel<F, RT, KS, RNPL, R, NW>>(lds);
  if (rc) return rc;
  TMOE_LAUNCH(TMOE_KERNEL_GATEUP, (gateup_kernel<F, RT, KS, RNPL, R, NW>), grid, dim3(64 * NW), lds, st, a);
  TMOE_LAUNCHED("gateup");
  return TMOE_OK;
}

static GateUpArgs gateup_args(const tmoe_moe_weights *W, const uint16_t *X, int64_t P, float clamp, float *Hout,
                              const FfnWs &fw, const int32_t *sorted_token) {
  const Geom gh = make_geom(W->hidden), gi = make_geom(W->inter);
  GateUpArgs ga{};
  ga.gate_p = W->gate_p;
  ga.up_p = W->up_p;
  ga.stride_gu = W->stride_gu;
  ga.gate_s = W->gate_s;
  ga.up_s = W->up_s;
  ga.X = X;
  ga.tiles = fw.tiles;
  ga.ntiles = fw.ntiles;
  ga.sorted_token = sorted_token;
  ga.h = Hout;
  ga.hf = fw.hf;
  ga.hmax = fw.hmax;
  ga.gx = gh;
  ga.gd = gi;
  ga.I = (int)W->inter;
  ga.clamp = clamp;
  return ga;
}

static int check_ffn_shapes(const tmoe_moe_weights *W) {
  const int64_t H = W->hidden, I = W->inter;
  const Geom gh = make_geom(H), gi = make_geom(I);
  if (!(gh.F == 13 && gh.r == 0 && gi.F == 3 && gi.r == 2 && H % 64 == 0 && I % 64 == 0))
    return fail(TMOE_E_UNSUPPORTED, "expert kernels are built for hidden 2048 and moe_intermediate 512");
  return TMOE_OK;
}

template <int R>
static int run_down_r(hipStream_t st, const DownArgs &da, int64_t max_tiles, int64_t H, bool walk) {
  const size_t lds = (size_t)2 * 17 * lds_row_bytes(da.slots);
  int rc = allow_lds<down_kernel<3, 2, R>>(lds);
  if (rc) return rc;
  TMOE_LAUNCH(TMOE_KERNEL_DOWN, (down_kernel<3, 2, R>),
              dim3(walk_grid(max_tiles * (H / 64 / R), walk)), dim3(256), lds, st, da);
  TMOE_LAUNCHED("down");
  return TMOE_OK;
}

static int run_down(hipStream_t st, const tmoe_moe_weights *W, const FfnWs &fw, int64_t P, int64_t max_tiles,
                    float *O) {
  const Geom gi = make_geom(W->inter);
  DownArgs da;
  da.down_p = W->down_p;
  da.stride_d = W->stride_d;
  da.down_s = W->down_s;
  da.hf = fw.hf;
  da.tiles = fw.tiles;
  da.ntiles = fw.ntiles;
  da.O = O;
  da.H = (int)W->hidden;
  da.I = (int)W->inter;
  da.slots = gi.slots;
  da.gd = gi;
  da.stream_w = P < 32 * W->n_experts;  // with many tiles per expert the caches serve the re-reads
  const bool walk = P < 4 * W->n_experts;
  if (P < 1024) return run_down_r<4>(st, da, max_tiles, W->hidden, walk);
  return run_down_r<8>(st, da, max_tiles, W->hidden, walk);  // 512 rows per item: h staged once for them
}

int launch_decode_tail(hipStream_t st, const tmoe_moe_weights *W, const uint16_t *X, int64_t T, float clamp,
                       const DecodeRoute &r, const FfnWs &fw, float *O, float *Y, const uint16_t *resid_in,
                       uint16_t *resid_out) {
  int rc = check_ffn_shapes(W);
  if (rc) return rc;
  const int64_t E = W->n_experts, H = W->hidden, I = W->inter;
  const int k = W->top_k;
  const int64_t P = T * k;
  if (T < 1 || T > kDecodeMaxT || k > 16 || E > 1024 || r.nb < 1 || r.nb > kRouterMaxSlots)
    return fail(TMOE_E_UNSUPPORTED, "decode path limits");
  const Geom gi = make_geom(I);
  GateUpArgs ga = gateup_args(W, X, P, clamp, nullptr, fw, r.sorted_token);
  ga.r = r;
  ga.r.tiles = fw.tiles;
  ga.r.ntiles = fw.ntiles;
  ga.r.pair_w = fw.pw;
  ga.T = (int)T;
  ga.E = (int)E;
  ga.k = k;
  const int64_t nx = P < E ? P : E;  // hit experts <= min(T k, E), one tile each
  if (E <= 256)
    rc = P <= 64 ? run_gateup<13, 0, 4, 4>(st, ga, nx, (int)I) : run_gateup<13, 0, 1, 4>(st, ga, nx, (int)I);
  else
    rc = P <= 64 ? run_gateup<13, 0, 4, 16>(st, ga, nx, (int)I) : run_gateup<13, 0, 1, 16>(st, ga, nx, (int)I);
  if (rc) return rc;

  if (P <= kDcMaxPairs) {
    DownCombineArgs da;
    da.down_p = W->down_p;
    da.stride_d = W->stride_d;
    da.down_s = W->down_s;
    da.hf = fw.hf;
    da.slots = gi.slots;
    da.I = (int)I;
    da.tiles = fw.tiles;
    da.ntiles = fw.ntiles;
    da.sorted_token = r.sorted_token;
    da.pair_w = fw.pw;
    da.P = (int)P;
    da.max_tiles = (int)nx;
    da.gd = gi;
    da.T = (int)T;
    da.H = (int)H;
    da.Y = Y;
    da.resid_in = resid_in;
    da.resid_out = resid_out;
    const size_t lds = (size_t)2 * P * gi.slots * 2;
    rc = allow_lds<down_combine_kernel<3, 2>>(lds);
    if (rc) return rc;
    TMOE_LAUNCH(TMOE_KERNEL_DOWN, (down_combine_kernel<3, 2>), dim3((unsigned)(H / 16)), dim3(64 * kDcWaves), lds,
                st, da);
    TMOE_LAUNCHED("down_combine");
    return TMOE_OK;
  }
  // more pairs: down over (tile, 64-row block) into O, then the combine
  rc = run_down(st, W, fw, P, nx, O);
  if (rc) return rc;
  return launch_combine(st, O, r.w, r.pos, T, k, H, Y, resid_in, resid_out);
}

int launch_ffn(hipStream_t st, const tmoe_moe_weights *W, const uint16_t *X, int64_t T, const int32_t *offsets,
               const int32_t *sorted_token, float clamp, float *O, float *Hout, const FfnWs &fw, bool tiles_ready) {
  int rc = check_ffn_shapes(W);
  if (rc) return rc;
  const int64_t E = W->n_experts, H = W->hidden, I = W->inter, P = T * W->top_k;
  const Geom gi = make_geom(I);
  const int64_t max_tiles = ffn_max_tiles(P, E);
  if (max_tiles > 0x7FFFFFFF || T > 0x7FFFFFFF) return fail(TMOE_E_UNSUPPORTED, "too many tokens");

  const bool tb = ffn_blocked(P, E, H, I);
  if (!tiles_ready && !tb) {
    TMOE_LAUNCH(TMOE_KERNEL_MAKE_TILES, make_tiles_kernel<16>, dim3(1), dim3(256), 0, st, offsets, (int)E, fw.tiles,
                fw.ntiles);
    TMOE_LAUNCHED("make_tiles");
  }

  GateUpArgs ga = gateup_args(W, X, P, clamp, Hout, fw, sorted_token);
  ga.offsets = offsets;
  if (tb) {
    // many pairs per expert: token-blocked (64 pairs x 256 rows per workgroup)
    if (!tiles_ready) {
      TMOE_LAUNCH(TMOE_KERNEL_MAKE_TILES, make_tiles_kernel<64>, dim3(1), dim3(256), 0, st, offsets, (int)E,
                  fw.blocks, fw.nblocks);
      TMOE_LAUNCHED("make_blocks");
    }
    GateUpArgs gb = ga;
    gb.tiles = fw.blocks;
    gb.ntiles = fw.nblocks;
    const size_t lds = (size_t)kTbDepth * kTbStepBytes;
    rc = allow_lds<gateup_tb_kernel<13>>(lds);
    if (rc) return rc;
    TMOE_LAUNCH(TMOE_KERNEL_GATEUP, gateup_tb_kernel<13>, dim3(tb_grid(ffn_max_blocks(P, E), (int)(I / kTbRows))),
                dim3(64 * kTbWaves), lds, st, gb);
    TMOE_LAUNCHED("gateup_tb");
  } else if (P <= 64)
    rc = run_gateup<13, 0, 4, 0>(st, ga, max_tiles, (int)I, P < 4 * E);
  else if (P < 1024)
    rc = run_gateup<13, 0, 1, 0, 1>(st, ga, max_tiles, (int)I, P < 4 * E);
  else
    rc = run_gateup<13, 0, 1, 0, 1, 8>(st, ga, max_tiles, (int)I, P < 4 * E);
  if (rc) return rc;

  if (tb) {
    // token-blocked down over the same 64-pair blocks
    DownArgs da;
    da.down_p = W->down_p;
    da.stride_d = W->stride_d;
    da.down_s = W->down_s;
    da.hf = fw.hf;
    da.hmax = fw.hmax;
    da.hgroups = (int)(I / kTbRows);
    da.tiles = fw.blocks;
    da.ntiles = fw.nblocks;
    da.O = O;
    da.H = (int)H;
    da.I = (int)I;
    da.slots = gi.slots;
    da.gd = gi;
    da.stream_w = 0;
    const size_t lds = (size_t)2 * 64 * lds_row_bytes(gi.slots);
    rc = allow_lds<down_tb_kernel<3, 2>>(lds);
    if (rc) return rc;
    TMOE_LAUNCH(TMOE_KERNEL_DOWN, (down_tb_kernel<3, 2>), dim3(dtb_grid()), dim3(64 * kDtbWaves), lds, st, da);
    TMOE_LAUNCHED("down_tb");
    return TMOE_OK;
  }
  return run_down(st, W, fw, P, max_tiles, O);
}

bool ffn_blocked(int64_t P, int64_t E, int64_t H, int64_t I) {
  return P >= 32 * E && I % kTbRows == 0 && I / kTbRows <= kTbMaxGroups && H == 16 * kDtbGroups * kDtbWaves * kDtbR;
}

size_t linear_ws_bytes(int64_t T, int64_t K) {
  (void)T;
  (void)K;
  return 0;
}

template <int F, int RT, int KS>
static int run_linear(hipStream_t st, const LinearArgs &a, int64_t ntok_tiles, int64_t nrt) {
  const int rs = lds_row_bytes(a.g.slots);
  size_t lds = (size_t)(a.zrow + 1) * rs + (KS > 1 ? 4 * 64 * 4 * 4 : 0);
  dim3 grid((unsigned)ntok_tiles, (unsigned)cdiv(nrt, 4 / KS));
  if (a.rows_x) grid = dim3((unsigned)cdiv(nrt, 4 / KS), (unsigned)ntok_tiles);
  if (grid.y > 65535) return fail(TMOE_E_UNSUPPORTED, "too many row tiles for one token tile grid");
  int rc = allow_lds<linear_kernel<F, RT, KS>>(lds);
  if (rc) return rc;
  TMOE_LAUNCH(TMOE_KERNEL_LINEAR, (linear_kernel<F, RT, KS>), grid, dim3(256), lds, st, a);
  TMOE_LAUNCHED("ternary_linear");
  return TMOE_OK;
}

int launch_linear(hipStream_t st, const uint8_t *Pt, const float *s, int64_t N, int64_t K, const uint16_t *X,
                  int64_t ldx, int64_t T, float *Y, int64_t ldy, void *ws) {
  (void)ws;
  const Geom g = make_geom(K);
  if ((size_t)17 * lds_row_bytes(g.slots) + 4096 > 160 * 1024) return fail(TMOE_E_UNSUPPORTED, "K too large");
  const int64_t nrt = cdiv(N, 16), ntt = cdiv(T, 16);
  if (ntt > 0x7FFFFFFF || nrt > 0x7FFFFFFF) return fail(TMOE_E_UNSUPPORTED, "too large");
  LinearArgs a;
  a.pt = Pt;
  a.s = s;
  a.X = X;
  a.Y = Y;
  a.T = T;
  a.N = N;
  a.ldx = ldx;
  a.ldy = ldy;
  a.g = g;
  a.contig = g.QS == 5 * g.Q && K % 8 == 0 && ldx % 8 == 0 && ((uintptr_t)X & 15) == 0;
  a.rows_x = ntt == 1;
  a.zrow = (int)(T < 16 ? T : 16);
  if (g.F == 13 && g.r == 0 && T <= 16 && nrt >= 8192 && a.contig) {
    // a streamed matrix: the rows alone fill the chip many times over
    const size_t lds = (size_t)(a.zrow + 1) * lds_row_bytes(g.slots);
    int rc = allow_lds<linear_stream_kernel>(lds);
    if (rc) return rc;
    const int64_t wgs = cdiv(nrt, 4) < kStreamWgs ? cdiv(nrt, 4) : kStreamWgs;
    TMOE_LAUNCH(TMOE_KERNEL_LINEAR, linear_stream_kernel, dim3((unsigned)wgs), dim3(256), lds, st, a);
    TMOE_LAUNCHED("ternary_linear_stream");
    return TMOE_OK;
  }
  // few tokens: K split over the four wavefronts (more workgroups for a few
  // thousand rows)
  const bool small = T <= 16;
  if (g.F == 13 && g.r == 0) return small ? run_linear<13, 0, 4>(st, a, ntt, nrt) : run_linear<13, 0, 1>(st, a, ntt, nrt);
  if (g.F == 3 && g.r == 2) return run_linear<3, 2, 1>(st, a, ntt, nrt);
  return run_linear<-1, 0, 1>(st, a, ntt, nrt);
}

int launch_linear3(hipStream_t st, const uint8_t *Pt, const float *s, int64_t N, int64_t K, const float *X, int64_t T,
                   float *Y, const uint16_t *resid_in, uint16_t *resid_out) {
  const Geom g = make_geom(K);
  if (!(g.F == 13 && g.r == 0 && g.QS == 5 * g.Q)) return fail(TMOE_E_UNSUPPORTED, "fp32-input linear needs K = 2048");
  const int64_t nrt = cdiv(N, 16), ntt = cdiv(T, kL3Tok);
  if (ntt > 0x7FFFFFFF || nrt > 0x7FFFFFFF) return fail(TMOE_E_UNSUPPORTED, "too large");
  Linear3Args a;
  a.pt = Pt;
  a.s = s;
  a.X = X;
  a.Y = Y;
  a.resid_in = resid_in;
  a.resid_out = resid_out;
  a.T = T;
  a.N = N;
  a.g = g;
  const size_t lds = (size_t)3 * (kL3Tok + 1) * lds_row_bytes(g.slots) + 4 * 64 * 4 * 4;
  if (T <= 16) {
    int rc = allow_lds<linear3_kernel<4>>(lds);
    if (rc) return rc;
    TMOE_LAUNCH(TMOE_KERNEL_LINEAR, linear3_kernel<4>, dim3((unsigned)ntt, (unsigned)nrt), dim3(256), lds, st, a);
  } else {
    int rc = allow_lds<linear3_kernel<1>>(lds);
    if (rc) return rc;
    TMOE_LAUNCH(TMOE_KERNEL_LINEAR, linear3_kernel<1>, dim3((unsigned)ntt, (unsigned)cdiv(nrt, 4)), dim3(256), lds, st,
                a);
  }
  TMOE_LAUNCHED("ternary_linear3");
  return TMOE_OK;
}

int launch_combine(hipStream_t st, const float *O, const float *w, const int32_t *pos, int64_t T, int k, int64_t H,
                   float *Y, const uint16_t *resid_in, uint16_t *resid_out) {
  if (T > 0x7FFFFFFF) return fail(TMOE_E_UNSUPPORTED, "T too large");
  const bool wide = T >= 1024;  // two columns per thread: 4096 tokens 50 -> 48.5 us
  const dim3 grid((unsigned)T, (unsigned)cdiv(H, wide ? 1024 : 512));
  if ((double)T * k * H * 4 > 64.0 * (1 << 20)) {  // expert outputs beyond 64 MB: stream them
    if (wide)
      TMOE_LAUNCH(TMOE_KERNEL_COMBINE, (combine_kernel<true, 2>), grid, dim3(128), 0, st, O, w, pos, k, (int)H, Y,
                  resid_in, resid_out);
    else
      TMOE_LAUNCH(TMOE_KERNEL_COMBINE, (combine_kernel<true, 1>), grid, dim3(128), 0, st, O, w, pos, k, (int)H, Y,
                  resid_in, resid_out);
  } else if (wide) {
    TMOE_LAUNCH(TMOE_KERNEL_COMBINE, (combine_kernel<false, 2>), grid, dim3(128), 0, st, O, w, pos, k, (int)H, Y,
                resid_in, resid_out);
  } else {
    TMOE_LAUNCH(TMOE_KERNEL_COMBINE, (combine_kernel<false, 1>), grid, dim3(128), 0, st, O, w, pos, k, (int)H, Y,
                resid_in, resid_out);
  }
  TMOE_LAUNCHED("combine");
  return TMOE_OK;
}

}  // namespace tmoe
