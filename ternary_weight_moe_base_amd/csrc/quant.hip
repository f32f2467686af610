// Weight preparation on the device: the synthetic weight source (Philox +
// Irwin-Hall), absmean ternarization with canonical 5-trit packing, unpacking,
// and the canonical <-> tiled layout conversions.
#include "common.h"

namespace tmoe {

// ------------------------------------------------------------- synthetic
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 64-bit
// multiplies (high and low halves) and xors, with a Weyl-sequence key schedule.
__device__ inline void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t lo0 = M0 * c[0], hi0 = __umul64hi(M0, c[0]);
    uint64_t lo1 = M1 * c[2], hi1 = __umul64hi(M1, c[2]);
    uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += W0;
    k1 += W1;
  }
}

__global__ void synth_ih12_kernel(uint64_t key0, uint64_t key1, uint64_t sid, uint64_t first, int64_t n, float mult,
                                  float *out) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint64_t c[4] = {first + (uint64_t)i, sid, 0, 0};
  philox4x64_10(c, key0, key1);
  int32_t s = 0;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    uint64_t w = c[j];
    s += (int32_t)(w & 0xFFFF) + (int32_t)((w >> 16) & 0xFFFF) + (int32_t)((w >> 32) & 0xFFFF) +
         (int32_t)(w >> 48);
  }
  float v = (float)(s - 393210) * 0x1p-16f;
  out[i] = v * mult;
}

int launch_synth_ih12(hipStream_t st, uint64_t key0, uint64_t key1, uint64_t sid, uint64_t first, int64_t n,
                      float mult, float *out) {
  const int B = 256;
  int64_t grid = cdiv(n, B);
  if (grid > 0x7FFFFFFF) return fail(TMOE_E_UNSUPPORTED, "n too large");
  hipLaunchKernelGGL(synth_ih12_kernel, dim3((unsigned)grid), dim3(B), 0, st, key0, key1, sid, first, n, mult, out);
  TMOE_LAUNCHED("synth_ih12");
  return TMOE_OK;
}

// ------------------------------------------------- ternarize + pack (device)
// Scales first: one lane per row, s = fp32(sum |w| / K) with the fp64 sum in
// index order, the same additions in the same order as the host definition,
// so s is bit-identical to it for any finite fp32 row. Each lane walks its own
// row, 64 inputs (two cache lines) in flight ahead of the additions when rows
// are 16-byte aligned.
__global__ __launch_bounds__(256) void absmean_rows_kernel(const float *W, int64_t R, int64_t K, float *S) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= R) return;
  const float *w = W + r * K;
  double acc = 0.0;
  int64_t i = 0;
  if ((K & 3) == 0 && ((uintptr_t)W & 15) == 0) {
    const float4 *w4 = reinterpret_cast<const float4 *>(w);
    for (; i + 64 <= K; i += 64) {
      float4 v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = w4[i / 4 + j];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        acc += fabs((double)v[j].x);
        acc += fabs((double)v[j].y);
        acc += fabs((double)v[j].z);
        acc += fabs((double)v[j].w);
      }
    }
  }
  for (; i < K; ++i) acc += fabs((double)w[i]);
  S[r] = K ? (float)(acc / (double)K) : 0.0f;
}

// Then one workgroup per row: trit = sign(w) if 2|w| > s else 0 (in fp64,
// exact), canonical base-3 bytes.
__global__ __launch_bounds__(256) void ternarize_pack_kernel(const float *W, int64_t K, uint8_t *P, int64_t ldp,
                                                             const float *S) {
  const int64_t r = blockIdx.x;
  const float *w = W + r * K;
  const double sd = (double)S[r];
  const int64_t Kb = (K + 4) / 5;
  for (int64_t j = threadIdx.x; j < Kb; j += 256) {
    int code = 0, p3 = 1;
#pragma unroll
    for (int q = 0; q < 5; ++q, p3 *= 3) {
      int64_t i = 5 * j + q;
      int d = 1;
      if (i < K) {
        float v = w[i];
        if (2.0 * fabs((double)v) > sd) d = v > 0.f ? 2 : 0;
      }
      code += d * p3;
    }
    P[r * ldp + j] = (uint8_t)code;
  }
}

int launch_ternarize_pack(hipStream_t st, const float *W, int64_t R, int64_t K, uint8_t *P, int64_t ldp, float *s) {
  if (R > 0x7FFFFFFF) return fail(TMOE_E_UNSUPPORTED, "R too large");
  hipLaunchKernelGGL(absmean_rows_kernel, dim3((unsigned)cdiv(R, 256)), dim3(256), 0, st, W, R, K, s);
  TMOE_LAUNCHED("absmean_rows");
  hipLaunchKernelGGL(ternarize_pack_kernel, dim3((unsigned)R), dim3(256), 0, st, W, K, P, ldp, s);
  TMOE_LAUNCHED("ternarize_pack");
  return TMOE_OK;
}

// ---------------------------------------------------------------- unpack
__device__ inline void decode5(int b, int8_t t[5]) {
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    t[q] = (int8_t)(b % 3 - 1);
    b /= 3;
  }
}

__global__ void unpack_kernel(const uint8_t *P, int64_t R, int64_t K, int64_t ldp, int8_t *T) {
  const int64_t Kb = (K + 4) / 5;
  int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= R * Kb) return;
  int64_t r = id / Kb, j = id % Kb;
  int8_t t[5];
  decode5(P[r * ldp + j], t);
#pragma unroll
  for (int q = 0; q < 5; ++q)
    if (5 * j + q < K) T[r * K + 5 * j + q] = t[q];
}

int launch_unpack(hipStream_t st, const uint8_t *P, int64_t R, int64_t K, int64_t ldp, int8_t *T) {
  int64_t n = R * ((K + 4) / 5);
  int64_t grid = cdiv(n, 256);
  if (grid > 0x7FFFFFFF) return fail(TMOE_E_UNSUPPORTED, "matrix too large");
  hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)grid), dim3(256), 0, st, P, R, K, ldp, T);
  TMOE_LAUNCHED("unpack");
  return TMOE_OK;
}

// ------------------------------------------------------- tiled conversions
// One thread per byte of the tiled image: tile, lane (row i = lane & 15,
// quarter g = lane >> 4) and quarter byte b are recovered from the offset; the
// byte's five trits are the input indices tiled_k(g, quarter, b, 0..4).
__device__ inline void tiled_coords(const Geom &g, int64_t off, int64_t &tile, int &lane, int &b) {
  tile = off / g.tile_bytes;
  int64_t o = off % g.tile_bytes;
  int64_t full = (int64_t)g.F * 512;
  if (o < full) {
    int s = (int)(o / 512);
    int w = (int)(o % 512);
    lane = w / 8;
    b = 8 * s + (w % 8);
    return;
  }
  int w = (int)(o - full);
  if (g.r >= 4) {
    if (w < 256) {
      lane = w / 4;
      b = 8 * g.F + (w % 4);
      return;
    }
    w -= 256;
    lane = w / 2;
    b = 8 * g.F + 4 + (w % 2);
    return;
  }
  lane = w / 2;
  b = 8 * g.F + (w % 2);
}

// canonical trit of input index k of a row (0 past K)
__device__ inline int canon_trit(const uint8_t *row, int64_t K, int64_t k) {
  if (k >= K) return 0;
  int b = row[k / 5];
  switch (k % 5) {
    case 4: b /= 81; break;
    case 3: b /= 27; break;
    case 2: b /= 9; break;
    case 1: b /= 3; break;
    default: break;
  }
  return b % 3 - 1;
}

__global__ void repack_tiled_kernel(const uint8_t *P, int64_t R, int64_t ldp, Geom g, int64_t total, uint8_t *Pt) {
  int64_t off = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (off >= total) return;
  int64_t tile;
  int lane, b;
  tiled_coords(g, off, tile, lane, b);
  const int64_t row = tile * 16 + (lane & 15);
  const int quarter = lane >> 4;
  int code = 0, p3 = 1;
#pragma unroll
  for (int q = 0; q < 5; ++q, p3 *= 3) {
    const int t = row < R ? canon_trit(P + row * ldp, g.K, tiled_k(g, quarter, b, q)) : 0;
    code += (t + 1) * p3;
  }
  Pt[off] = (uint8_t)code;
}

__global__ void unpack_tiled_kernel(const uint8_t *Pt, int64_t R, Geom g, int64_t total, int8_t *T) {
  int64_t off = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (off >= total) return;
  int64_t tile;
  int lane, b;
  tiled_coords(g, off, tile, lane, b);
  const int64_t row = tile * 16 + (lane & 15);
  if (row >= R) return;
  const int quarter = lane >> 4;
  int8_t t[5];
  const int v = Pt[off];
  decode5(v > 242 ? 121 : v, t);
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    const int64_t k = tiled_k(g, quarter, b, q);
    if (k < g.K) T[row * g.K + k] = t[q];
  }
}

int launch_repack_tiled(hipStream_t st, const uint8_t *P, int64_t R, int64_t K, int64_t ldp, uint8_t *Pt) {
  Geom g = make_geom(K);
  int64_t total = cdiv(R, 16) * g.tile_bytes;
  int64_t grid = cdiv(total, 256);
  if (grid > 0x7FFFFFFF) return fail(TMOE_E_UNSUPPORTED, "matrix too large");
  hipLaunchKernelGGL(repack_tiled_kernel, dim3((unsigned)grid), dim3(256), 0, st, P, R, ldp, g, total, Pt);
  TMOE_LAUNCHED("repack_tiled");
  return TMOE_OK;
}

int launch_unpack_tiled(hipStream_t st, const uint8_t *Pt, int64_t R, int64_t K, int8_t *T) {
  Geom g = make_geom(K);
  int64_t total = cdiv(R, 16) * g.tile_bytes;
  int64_t grid = cdiv(total, 256);
  if (grid > 0x7FFFFFFF) return fail(TMOE_E_UNSUPPORTED, "matrix too large");
  hipLaunchKernelGGL(unpack_tiled_kernel, dim3((unsigned)grid), dim3(256), 0, st, Pt, R, g, total, T);
  TMOE_LAUNCHED("unpack_tiled");
  return TMOE_OK;
}

}  // namespace tmoe
