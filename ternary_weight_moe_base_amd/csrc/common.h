// Internal declarations shared by the host and device sources of libtmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "tmoe.h"

namespace tmoe {

// ---------------------------------------------------------------- errors
// Records a thread-local message and returns `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int hip_fail(hipError_t e, const char *what);

#define TMOE_HIP(expr)                                 \
  do {                                                 \
    hipError_t e_ = (expr);                            \
    if (e_ != hipSuccess) return ::tmoe::hip_fail(e_, #expr); \
  } while (0)

// Launch check: reports a launch-configuration error of the preceding launch.
#define TMOE_LAUNCHED(name)                                \
  do {                                                     \
    hipError_t e_ = hipGetLastError();                     \
    if (e_ != hipSuccess) return ::tmoe::hip_fail(e_, name); \
  } while (0)

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ------------------------------------------------------- tiled weight layout
// A weight matrix [R][K] is stored as ceil(R/16) tiles of 16 rows. Each row's
// ceil(K/5) canonical bytes are split in four quarters of Q bytes (Q even);
// quarter g of tile row i belongs to lane i + 16g of the wavefront that
// multiplies the tile. A lane's quarter is consumed in "steps" of 8 bytes
// (4 byte pairs -> 20 bf16 pair-words -> 5 MFMA 16x16x32 operands) and a tail
// of r = Q mod 8 bytes (0, 2, 4 or 6). Inside a tile:
//   full step s < F : offset s*512 + lane*8 + b      (b < 8)
//   tail dword part : offset F*512 + lane*4 + b      (r >= 4, b < 4)
//   tail short part : offset F*512 + (r>=4 ? 256 : 0) + lane*2 + b (r odd pair)
// Every offset is a contiguous 512/256/128-byte run per wavefront load.
struct Geom {
  int64_t K;      // real input width
  int64_t Kb;     // canonical bytes per row = ceil(K/5)
  int32_t Q;      // bytes per quarter (even)
  int32_t F;      // full 8-byte steps per quarter
  int32_t r;      // tail bytes per quarter (0, 2, 4, 6)
  int32_t tailM;  // MFMAs for the tail (0, 2, 3, 4)
  int32_t M;      // MFMAs per 16-row tile over the whole K = 5F + tailM
  int32_t slots;  // operand slots per token = 4 quarters * M * 8
  int64_t tile_bytes;  // 64 * Q
};

__host__ __device__ inline Geom make_geom(int64_t K) {
  Geom g;
  g.K = K;
  g.Kb = (K + 4) / 5;
  int64_t q = (g.Kb + 3) / 4;
  q += (q & 1);
  if (q < 2) q = 2;
  g.Q = (int32_t)q;
  g.F = g.Q / 8;
  g.r = g.Q % 8;
  g.tailM = g.r == 0 ? 0 : (5 * (g.r / 2) + 3) / 4;
  g.M = 5 * g.F + g.tailM;
  g.slots = 32 * g.M;
  g.tile_bytes = 64 * (int64_t)g.Q;
  return g;
}

// Offset, inside a tile, of byte b (0 <= b < Q) of the quarter read by `lane`.
__host__ __device__ inline int64_t tile_offset(const Geom &g, int lane, int b) {
  int full = 8 * g.F;
  if (b < full) return (int64_t)(b / 8) * 512 + lane * 8 + (b % 8);
  int tb = b - full;
  int64_t base = (int64_t)g.F * 512;
  if (g.r >= 4) {
    if (tb < 4) return base + lane * 4 + tb;
    return base + 256 + lane * 2 + (tb - 4);
  }
  return base + lane * 2 + tb;
}

// Input index K of operand slot `slot` (0 <= slot < g.slots), or -1 for a pad
// slot. Slot = (quarter * M + mfma) * 8 + e: element e of the 8-wide operand
// of MFMA `mfma` for the lanes of quarter `quarter`. Element e is half (e & 1)
// of pair-word i = e >> 1; pair-word u = 4 * mfma' + i counts the 5 base-3
// digits q of byte pairs p = u / 5 (q = u % 5) of the step; half 0 is the
// pair's first byte.
__host__ __device__ inline int64_t slot_to_k(const Geom &g, int slot) {
  int e = slot & 7;
  int mi = (slot >> 3) % g.M;
  int quarter = (slot >> 3) / g.M;
  int i = e >> 1, h = e & 1;
  int b, q;
  if (mi < 5 * g.F) {
    int s = mi / 5, m = mi % 5;
    int u = 4 * m + i;
    b = 8 * s + 2 * (u / 5) + h;
    q = u % 5;
  } else {
    int u = 4 * (mi - 5 * g.F) + i;
    if (u >= 5 * (g.r / 2)) return -1;
    b = 8 * g.F + 2 * (u / 5) + h;
    q = u % 5;
  }
  int64_t k = 5 * ((int64_t)quarter * g.Q + b) + q;
  return k < g.K ? k : -1;
}

// ---------------------------------------------------------------- launchers
// (defined in the .hip files; host code calls them after validating arguments)
int launch_synth_ih12(hipStream_t st, uint64_t key0, uint64_t key1, uint64_t sid, uint64_t first, int64_t n,
                      float mult, float *out);
int launch_ternarize_pack(hipStream_t st, const float *W, int64_t R, int64_t K, uint8_t *P, int64_t ldp, float *s);
int launch_unpack(hipStream_t st, const uint8_t *P, int64_t R, int64_t K, int64_t ldp, int8_t *T);
int launch_repack_tiled(hipStream_t st, const uint8_t *P, int64_t R, int64_t K, int64_t ldp, uint8_t *Pt);
int launch_unpack_tiled(hipStream_t st, const uint8_t *Pt, int64_t R, int64_t K, int8_t *T);

struct RouterWs {
  float *wl1;         // [E]    L1 norms of router rows
  float *logits;      // [T][E] fp32 logits
  int32_t *fix_count; // [1]
  int32_t *fix_list;  // [T]
};
size_t router_ws_bytes(int64_t T, int64_t E);
RouterWs router_ws_carve(void *ws, int64_t T, int64_t E);
int launch_router(hipStream_t st, const uint16_t *X, int64_t T, int64_t H, const float *Wr, const float *bias,
                  int64_t E, int k, int32_t *idx, float *w, float *logits_out, int32_t *n_fixup, const RouterWs &rw);

struct GroupWs {
  int32_t *bcount;  // [nb][E]
  int32_t *bbase;   // [nb][E]
};
size_t group_ws_bytes(int64_t T, int k, int64_t E);
GroupWs group_ws_carve(void *ws, int64_t T, int k, int64_t E);
int launch_group(hipStream_t st, const int32_t *idx, int64_t T, int k, int64_t E, int32_t *counts, int32_t *offsets,
                 int32_t *sorted_token, int32_t *sorted_slot, int32_t *pos, const GroupWs &gw);

struct FfnWs {
  int32_t *tiles;    // [max_tiles][4]: expert, start, count, 0
  int32_t *ntiles;   // [1]
  uint16_t *xp;      // [T][slots_H] bf16, permuted activations
  float *h;          // [T*k][I] fp32 (natural order), when the caller gives none
  uint16_t *hp;      // [2][T*k][slots_I] fp16 hi / lo parts, permuted
  int32_t *hexp;     // [T*k] power-of-two scale of each h row before the fp16 split
};
int64_t ffn_max_tiles(int64_t pairs, int64_t E);
size_t ffn_ws_bytes(int64_t T, int k, int64_t E, int64_t H, int64_t I);
FfnWs ffn_ws_carve(void *ws, int64_t T, int k, int64_t E, int64_t H, int64_t I);
int launch_ffn(hipStream_t st, const tmoe_moe_weights *W, const uint16_t *X, int64_t T, const int32_t *offsets,
               const int32_t *sorted_token, float clamp, float *O, float *Hout, const FfnWs &fw);

size_t linear_ws_bytes(int64_t T, int64_t K);
int launch_linear(hipStream_t st, const uint8_t *Pt, const float *s, int64_t N, int64_t K, const uint16_t *X,
                  int64_t ldx, int64_t T, float *Y, int64_t ldy, void *ws);

int launch_combine(hipStream_t st, const float *O, const float *w, const int32_t *pos, int64_t T, int k, int64_t H,
                   float *Y, const uint16_t *resid_in, uint16_t *resid_out);

}  // namespace tmoe
