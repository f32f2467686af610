// Internal declarations shared by the host and device sources of libtmoe.
#pragma once

#include <atomic>

#include <hip/hip_ext.h>
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
// A weight matrix [R][K] is stored as ceil(R/16) tiles of 16 rows. Each row is
// split in four quarters; quarter g holds the 5Q input indices
// [5Qg, 5Qg + 5Q) in Q bytes (Q even, 4Q >= ceil(K/5)); indices >= K are
// zero trits. Quarter g of tile row i belongs to lane i + 16g of the
// wavefront that multiplies the tile. A lane consumes its Q bytes in F "steps"
// of 8 bytes and a tail of r = Q mod 8 bytes (0, 2, 4 or 6). Inside a step
// (or the tail), byte 2p + h (pair p, half h) holds, as base-3 digit q (digit
// = trit + 1, weight 3^q), the trit of input index
//     5Qg + 40s + 10p + 2q + h        (s = step; the tail counts as step F).
// The packed-fp16 decoder turns byte pair p into five "pair-words" u = 5p + q
// holding the two trits of indices 40s + 2u + {0, 1}: MFMA m of the step takes
// pair-words 4m..4m+3, i.e. the 8 consecutive input indices 5Qg + 8(5s+m) + e,
// e = 0..7. The activation operand is therefore the input row itself, laid out
// per quarter: operand position g*QS + j (QS = 8M, M = MFMAs per quarter) holds
// input 5Qg + j for j < 5Q (zero beyond 5Q or K).
// Tile byte order (each wavefront load is one contiguous run):
//   full step s < F : offset s*512 + lane*8 + b      (b < 8)
//   tail dword part : offset F*512 + lane*4 + b      (r >= 4, b < 4)
//   tail short part : offset F*512 + (r>=4 ? 256 : 0) + lane*2 + b
struct Geom {
  int64_t K;      // real input width
  int64_t Kb;     // canonical bytes per row = ceil(K/5)
  int32_t Q;      // bytes per quarter (even)
  int32_t F;      // full 8-byte steps per quarter
  int32_t r;      // tail bytes per quarter (0, 2, 4, 6)
  int32_t tailM;  // MFMAs for the tail (0, 2, 3, 4)
  int32_t M;      // MFMAs per quarter = 5F + tailM
  int32_t QS;     // operand positions per quarter = 8M (>= 5Q)
  int32_t slots;  // operand positions per row = 4 QS
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
  g.QS = 8 * g.M;
  g.slots = 4 * g.QS;
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

// Input index held by digit q of byte b of quarter `quarter` (>= K: a zero trit).
__host__ __device__ inline int64_t tiled_k(const Geom &g, int quarter, int b, int q) {
  const int full = 8 * g.F;
  const int s = b < full ? b / 8 : g.F;
  const int bb = b < full ? b % 8 : b - full;
  return 5LL * g.Q * quarter + 40 * s + 10 * (bb >> 1) + 2 * q + (bb & 1);
}

// Input index of operand position j (0 <= j < QS) of quarter `quarter`, or -1.
__host__ __device__ inline int64_t operand_k(const Geom &g, int quarter, int j) {
  if (j >= 5 * g.Q) return -1;
  const int64_t k = 5LL * g.Q * quarter + j;
  return k < g.K ? k : -1;
}

// ------------------------------------------------------------ kernel timing
// When a tmoe_profile_begin window selects kernel `kid`, hands out the next
// event pair (and returns true); the launch then records them itself.
bool prof_events(int kid, hipEvent_t *start, hipEvent_t *stop);

// Launch that, under a profiling window for `kid`, carries start/stop events
// recorded by the dispatch itself (hipExtLaunchKernelGGL).
// A timed launch first waits for the stream to drain, so that its events
// bracket the kernel alone (no queued predecessor inside the interval).
#define TMOE_LAUNCH(kid, kernel, grid, block, lds, st, ...)                              \
  do {                                                                                 \
    hipEvent_t ev0_, ev1_;                                                             \
    if (::tmoe::prof_events(kid, &ev0_, &ev1_)) {                                      \
      (void)hipStreamSynchronize(st);                                                  \
      hipExtLaunchKernelGGL(kernel, grid, block, lds, st, ev0_, ev1_, 0, __VA_ARGS__); \
    } else {                                                                           \
      hipLaunchKernelGGL(kernel, grid, block, lds, st, __VA_ARGS__);                   \
    }                                                                                  \
  } while (0)

// Kernels using more than 64 KiB of LDS opt in once per kernel (gfx950 has 160 KiB;
// each such kernel always asks for the same size). Concurrent first calls may
// both set the attribute, which is idempotent.
template <auto Kern>
inline int allow_lds(size_t bytes) {
  static std::atomic<bool> done{false};  // one flag per kernel instantiation
  if (bytes <= 65536 || done.load(std::memory_order_acquire)) return TMOE_OK;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(Kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)bytes);
  if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute(MaxDynamicSharedMemorySize)");
  done.store(true, std::memory_order_release);
  return TMOE_OK;
}

// ---------------------------------------------------------------- launchers
// (defined in the .hip files; host code calls them after validating arguments)
int launch_synth_ih12(hipStream_t st, uint64_t key0, uint64_t key1, uint64_t sid, uint64_t first, int64_t n,
                      float mult, float *out);
int launch_ternarize_pack(hipStream_t st, const float *W, int64_t R, int64_t K, uint8_t *P, int64_t ldp, float *s);
int launch_unpack(hipStream_t st, const uint8_t *P, int64_t R, int64_t K, int64_t ldp, int8_t *T);
int launch_repack_tiled(hipStream_t st, const uint8_t *P, int64_t R, int64_t K, int64_t ldp, uint8_t *Pt);
int launch_unpack_tiled(hipStream_t st, const uint8_t *Pt, int64_t R, int64_t K, int8_t *T);

// Per-token error-bound inputs: bnd[t * nb + b] holds the bits of workgroup
// b's maximum over its experts of (sum_i |x_i w_ei| + |b_e|) (fp64 >= 0), one
// plain store per slot (no atomics, nothing to clear); a token's bound is the
// maximum of its nb slots. nb = experts / 4 (VALU logits) or / 16 (matrix cores).
struct RouterWs {
  uint64_t *bnd;     // [T][nb], capacity T * ceil(E / 4)
  double *lg;        // [T][E] fp64 logits (the bf16 matrix-core candidate logits on that path)
  // from 1024 tokens on (the bf16 candidate path):
  uint16_t *parts;   // [2][E][H] bf16 parts w1, w2 of the router rows (H <= 4096)
  uint64_t *wmax;    // [2][ceil(E / 4)] largest row norm and |bias| per split workgroup
  double *wnorm;     // [E] row norms |w_e|_2
  float *part;       // [4][T][E] fp32 slice sums of the candidate logits
};
// H: the router's hidden size (the bf16 parts of its rows take 4 E H bytes from 1024 tokens on).
size_t router_ws_bytes(int64_t T, int64_t E, int64_t H);
RouterWs router_ws_carve(void *ws, int64_t T, int64_t E, int64_t H);
constexpr int64_t kRouterMaxH = 4096;  // largest router hidden size (sizes tmoe_router_workspace_bytes)
// bound slots per token of the fp64 logits kernel: one per four experts, E <= 1024
constexpr int kRouterMaxSlots = 256;
// Logits (fp64 VALU for T <= 64, fp64 matrix cores above) and the certified
// top-k with its double-double fall-back (two kernels).
int launch_router(hipStream_t st, const uint16_t *X, int64_t T, int64_t H, const float *Wr, const float *bias,
                  int64_t E, int k, int32_t *idx, float *w, float *logits_out, int32_t *n_fixup, const RouterWs &rw);
// Logits and per-token bound slots only (the decode layer path, T <= 3, certifies
// the top-k in the gate/up kernel's prologue). Returns the error-bound depth in
// *depth and the bound slots per token in *nb.
int launch_router_logits(hipStream_t st, const uint16_t *X, int64_t T, int64_t H, const float *Wr, const float *bias,
                         int64_t E, const RouterWs &rw, int *depth, int *nb);
// Decode path (T <= kDecodeMaxT): every (token, slot) pair of an expert fits one work tile.
constexpr int kDecodeMaxT = 16;
// Token counts that take the three-kernel decode path in the layer call.
constexpr int kDecodePathMaxT = 3;  // measured: from 4 tokens on the batched path is faster

struct GroupWs {
  int32_t *bcount;  // [nb][E]
  int32_t *bbase;   // [nb][E]
};
size_t group_ws_bytes(int64_t T, int k, int64_t E);
GroupWs group_ws_carve(void *ws, int64_t T, int k, int64_t E);
// tiles / ntiles (may be null): also write the work tiles (<= `tile` pairs of one expert each)
int launch_group(hipStream_t st, const int32_t *idx, int64_t T, int k, int64_t E, int32_t *counts, int32_t *offsets,
                 int32_t *sorted_token, int32_t *sorted_slot, int32_t *pos, const GroupWs &gw, int32_t *tiles,
                 int32_t *ntiles, int tile);
// Whether the expert kernels take the token-blocked form (64-pair blocks) for P pairs.
bool ffn_blocked(int64_t P, int64_t E, int64_t H, int64_t I);

struct FfnWs {
  int32_t *tiles;    // [max_tiles][4]: expert, start, count, 0
  int32_t *ntiles;   // [1]
  float *hf;         // [T*k][I] fp32 h of each grouped pair (gate/up writes it; the down
                     // kernels split it into scaled fp16 parts while staging)
  float *pw;         // [T*k] routing weight of each grouped pair (decode path)
  int32_t *blocks;   // [max_blocks][4]: expert, start, count (<= 64), 0 (token-blocked gate/up)
  int32_t *nblocks;  // [1]
  uint32_t *hmax;    // [T*k][4] largest |h| (fp32 bits) of each pair per gate/up row group (token-blocked path)
};
int64_t ffn_max_tiles(int64_t pairs, int64_t E);
size_t ffn_ws_bytes(int64_t T, int k, int64_t E, int64_t H, int64_t I);
FfnWs ffn_ws_carve(void *ws, int64_t T, int k, int64_t E, int64_t H, int64_t I);
// Grouped expert FFN (gate/up + SiLU/clamp, down) from grouping offsets;
// tiles_ready: the grouping already wrote the work tiles the expert kernels
// take: fw.blocks / fw.nblocks (64 pairs) when ffn_blocked, else fw.tiles /
// fw.ntiles (16 pairs).
int launch_ffn(hipStream_t st, const tmoe_moe_weights *W, const uint16_t *X, int64_t T, const int32_t *offsets,
               const int32_t *sorted_token, float clamp, float *O, float *Hout, const FfnWs &fw, bool tiles_ready);

// Decode layer tail (T <= kDecodeMaxT): gate/up whose prologue certifies the
// top-k of every token from the fp64 logits and groups the pairs (workgroup
// (0, 0) publishes idx, w, grouping arrays and work tiles), then, for at most
// kDcMaxPairs pairs, down with the weighted combine (+ residual) fused, else
// down into O and the combine. The per-token bound slots are cleared for the
// next call.
// 1.01 gamma_d (gamma_d = d u / (1 - d u), u = 2^-53): the factor of the fp64
// logits' error bound for summation depth d, formed once on the host (the
// same IEEE operations in the same order as a device-side evaluation).
inline double topk_bound_scale(int d) {
  const double u = 0x1p-53;
  return 1.01 * ((double)d * u / (1.0 - (double)d * u));
}

struct DecodeRoute {
  const double *lg;
  const uint64_t *bnd;
  int depth, nb;  // error-bound depth; bound slots per token
  double bscale;  // topk_bound_scale(depth)
  const float *Wr, *bias;
  int32_t *idx, *n_fixup, *sorted_token, *sorted_slot, *pos;
  float *w;
  int32_t *tiles, *ntiles;  // set by launch_decode_tail (FFN workspace)
  float *pair_w;            // [T*k] routing weight of each grouped pair (FFN workspace)
};
// O [T*k][H] is used (and must exist) only when T*k > kDcMaxPairs.
constexpr int kDcMaxPairs = 32;
int launch_decode_tail(hipStream_t st, const tmoe_moe_weights *W, const uint16_t *X, int64_t T, float clamp,
                       const DecodeRoute &r, const FfnWs &fw, float *O, float *Y, const uint16_t *resid_in,
                       uint16_t *resid_out);

size_t linear_ws_bytes(int64_t T, int64_t K);
int launch_linear(hipStream_t st, const uint8_t *Pt, const float *s, int64_t N, int64_t K, const uint16_t *X,
                  int64_t ldx, int64_t T, float *Y, int64_t ldy, void *ws);

// Attention half (attention.hip): workspace bytes and the launch sequence
// (q/k/v linear, rotary + cache append, split attention, merge, o linear + residual).
int attn_nsplit(int64_t T, int nkv);
size_t attn_ws_bytes(int64_t T, int nh, int nkv, int hd);
int launch_attention(hipStream_t st, const tmoe_attn_weights &W, const uint16_t *X, int64_t T, int64_t pos0,
                     float *kc, float *vc, int64_t cap, float *O, uint16_t *X_out, void *ws);
// Ternary linear over fp32 inputs (three exact bf16 parts), K = 2048, optional bf16 residual.
int launch_linear3(hipStream_t st, const uint8_t *Pt, const float *s, int64_t N, int64_t K, const float *X, int64_t T,
                   float *Y, const uint16_t *resid_in, uint16_t *resid_out);
int launch_combine(hipStream_t st, const float *O, const float *w, const int32_t *pos, int64_t T, int k, int64_t H,
                   float *Y, const uint16_t *resid_in, uint16_t *resid_out);

// The whole layer (host_api.cpp): argument checks and the launch sequence of
// tmoe_moe_forward on a given workspace, and that workspace's size.
int moe_forward_impl(void *stream, const tmoe_moe_weights *W, const uint16_t *X, int64_t T, float *Y,
                     const tmoe_moe_options *opt, void *ws, size_t ws_bytes);
int moe_workspace_total(int64_t T, const tmoe_moe_weights *W, size_t *out);

// LM head (lmhead.hip)
size_t lmh_ws_bytes(int64_t T, int64_t V, int k);
int launch_lm_head(hipStream_t st, const uint16_t *X, int64_t T, int64_t H, const uint16_t *W, int64_t V, int k,
                   int32_t *idx, float *val, float *logits, int32_t *n_fixup, void *ws);

}  // namespace tmoe
