// Host side of libtmoe: status handling, the offline weight steps on the
// host (absmean ternarization, 5-trit packing), and the argument checks of
// every device entry point before its kernels are enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "common.h"

namespace tmoe {

static thread_local char g_err[512];

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = 0; }

int hip_fail(hipError_t e, const char *what) {
  return fail(TMOE_E_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

// ------------------------------------------------------------ kernel timing
// The measurement window of the calling thread (launches from other threads
// never see it).
struct ProfWindow {
  int kernel = 0, cap = 0, n = 0;
  hipEvent_t *start = nullptr, *stop = nullptr;
};
static thread_local ProfWindow g_prof;

bool prof_events(int kid, hipEvent_t *start, hipEvent_t *stop) {
  if (g_prof.kernel != kid || g_prof.n >= g_prof.cap) return false;
  *start = g_prof.start[g_prof.n];
  *stop = g_prof.stop[g_prof.n];
  ++g_prof.n;
  return true;
}

static void prof_free() {
  for (int i = 0; i < g_prof.cap; ++i) {
    if (g_prof.start && g_prof.start[i]) hipEventDestroy(g_prof.start[i]);
    if (g_prof.stop && g_prof.stop[i]) hipEventDestroy(g_prof.stop[i]);
  }
  delete[] g_prof.start;
  delete[] g_prof.stop;
  g_prof = {};
}

}  // namespace tmoe

using namespace tmoe;

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

extern "C" {

const char *tmoe_status_str(int s) {
  switch (s) {
    case TMOE_OK: return "TMOE_OK";
    case TMOE_E_ARG: return "TMOE_E_ARG";
    case TMOE_E_SHAPE: return "TMOE_E_SHAPE";
    case TMOE_E_ALIGN: return "TMOE_E_ALIGN";
    case TMOE_E_BADPACK: return "TMOE_E_BADPACK";
    case TMOE_E_WORKSPACE: return "TMOE_E_WORKSPACE";
    case TMOE_E_UNSUPPORTED: return "TMOE_E_UNSUPPORTED";
    case TMOE_E_HIP: return "TMOE_E_HIP";
    default: return "TMOE_E_UNKNOWN";
  }
}

const char *tmoe_last_error(void) { return g_err; }

int tmoe_version(void) { return 100; }

// ------------------------------------------------------------- host weights
int tmoe_ternarize_absmean_host(const float *W, int64_t R, int64_t K, int8_t *T, float *s) {
  clear_error();
  REQUIRE(R >= 0 && K >= 0, TMOE_E_ARG, "negative size R=%lld K=%lld", (long long)R, (long long)K);
  if (R == 0) return TMOE_OK;
  REQUIRE(W && T && s, TMOE_E_ARG, "null pointer");
  for (int64_t i = 0; i < R * K; ++i)
    REQUIRE(isfinite(W[i]), TMOE_E_ARG, "W[%lld] is not finite", (long long)i);
  for (int64_t r = 0; r < R; ++r) {
    const float *w = W + r * K;
    double acc = 0.0;  // index order
    for (int64_t i = 0; i < K; ++i) acc += fabs((double)w[i]);
    float sc = K ? (float)(acc / (double)K) : 0.0f;
    s[r] = sc;
    for (int64_t i = 0; i < K; ++i) {
      double a = fabs((double)w[i]);
      T[r * K + i] = (2.0 * a > (double)sc) ? (w[i] > 0 ? 1 : -1) : 0;
    }
  }
  return TMOE_OK;
}

int tmoe_pack_host(const int8_t *T, int64_t R, int64_t K, uint8_t *P, int64_t ldp) {
  clear_error();
  REQUIRE(R >= 0 && K >= 0, TMOE_E_ARG, "negative size");
  const int64_t Kb = (K + 4) / 5;
  REQUIRE(ldp >= Kb, TMOE_E_SHAPE, "ldp=%lld < ceil(K/5)=%lld", (long long)ldp, (long long)Kb);
  if (R == 0 || K == 0) return TMOE_OK;
  REQUIRE(T && P, TMOE_E_ARG, "null pointer");
  for (int64_t i = 0; i < R * K; ++i)
    REQUIRE(T[i] >= -1 && T[i] <= 1, TMOE_E_ARG, "trit T[%lld]=%d not in {-1,0,1}", (long long)i, (int)T[i]);
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t j = 0; j < Kb; ++j) {
      int code = 0, p3 = 1;
      for (int q = 0; q < 5; ++q, p3 *= 3) {
        int64_t i = 5 * j + q;
        int d = (i < K) ? T[r * K + i] + 1 : 1;
        code += d * p3;
      }
      P[r * ldp + j] = (uint8_t)code;
    }
  }
  return TMOE_OK;
}

int tmoe_unpack_host(const uint8_t *P, int64_t R, int64_t K, int64_t ldp, int8_t *T) {
  clear_error();
  REQUIRE(R >= 0 && K >= 0, TMOE_E_ARG, "negative size");
  const int64_t Kb = (K + 4) / 5;
  REQUIRE(ldp >= Kb, TMOE_E_SHAPE, "ldp < ceil(K/5)");
  if (R == 0 || K == 0) return TMOE_OK;
  REQUIRE(T && P, TMOE_E_ARG, "null pointer");
  for (int64_t r = 0; r < R; ++r)
    for (int64_t j = 0; j < Kb; ++j) {
      int b = P[r * ldp + j];
      REQUIRE(b <= 242, TMOE_E_BADPACK, "byte %d at row %lld col %lld", b, (long long)r, (long long)j);
      for (int q = 0; q < 5; ++q) {
        int64_t i = 5 * j + q;
        if (i < K) T[r * K + i] = (int8_t)(b % 3 - 1);
        b /= 3;
      }
    }
  return TMOE_OK;
}

int tmoe_validate_packed_host(const uint8_t *P, int64_t R, int64_t K, int64_t ldp, int64_t *n_bad) {
  clear_error();
  REQUIRE(R >= 0 && K >= 0 && n_bad, TMOE_E_ARG, "bad argument");
  const int64_t Kb = (K + 4) / 5;
  REQUIRE(ldp >= Kb, TMOE_E_SHAPE, "ldp < ceil(K/5)");
  *n_bad = 0;
  if (R == 0 || K == 0) return TMOE_OK;
  REQUIRE(P, TMOE_E_ARG, "null pointer");
  int64_t bad = 0;
  for (int64_t r = 0; r < R; ++r)
    for (int64_t j = 0; j < Kb; ++j) bad += P[r * ldp + j] > 242;
  *n_bad = bad;
  return bad ? fail(TMOE_E_BADPACK, "%lld invalid bytes", (long long)bad) : TMOE_OK;
}

int64_t tmoe_tiled_bytes(int64_t R, int64_t K) {
  if (R <= 0 || K <= 0) return 0;
  return cdiv(R, 16) * make_geom(K).tile_bytes;
}

// ------------------------------------------------------------ device weights
int tmoe_synth_ih12(void *stream, uint64_t key0, uint64_t key1, uint64_t sid, uint64_t first, int64_t n, float mult,
                    float *out) {
  clear_error();
  REQUIRE(n >= 0, TMOE_E_ARG, "negative n");
  if (n == 0) return TMOE_OK;
  REQUIRE(out, TMOE_E_ARG, "null out");
  REQUIRE(aligned4(out), TMOE_E_ALIGN, "out not 4-byte aligned");
  return launch_synth_ih12((hipStream_t)stream, key0, key1, sid, first, n, mult, out);
}

int tmoe_ternarize_pack(void *stream, const float *W, int64_t R, int64_t K, uint8_t *P, int64_t ldp, float *s) {
  clear_error();
  REQUIRE(R >= 0 && K >= 0, TMOE_E_ARG, "negative size");
  REQUIRE(ldp >= (K + 4) / 5, TMOE_E_SHAPE, "ldp < ceil(K/5)");
  if (R == 0) return TMOE_OK;
  REQUIRE(W && P && s, TMOE_E_ARG, "null pointer");
  REQUIRE(aligned4(W) && aligned4(s), TMOE_E_ALIGN, "W and s must be 4-byte aligned");
  return launch_ternarize_pack((hipStream_t)stream, W, R, K, P, ldp, s);
}

int tmoe_unpack(void *stream, const uint8_t *P, int64_t R, int64_t K, int64_t ldp, int8_t *T) {
  clear_error();
  REQUIRE(R >= 0 && K >= 0, TMOE_E_ARG, "negative size");
  REQUIRE(ldp >= (K + 4) / 5, TMOE_E_SHAPE, "ldp < ceil(K/5)");
  if (R == 0 || K == 0) return TMOE_OK;
  REQUIRE(P && T, TMOE_E_ARG, "null pointer");
  return launch_unpack((hipStream_t)stream, P, R, K, ldp, T);
}

int tmoe_repack_tiled(void *stream, const uint8_t *P, int64_t R, int64_t K, int64_t ldp, uint8_t *Pt) {
  clear_error();
  REQUIRE(R >= 0 && K >= 0, TMOE_E_ARG, "negative size");
  REQUIRE(ldp >= (K + 4) / 5, TMOE_E_SHAPE, "ldp < ceil(K/5)");
  if (R == 0 || K == 0) return TMOE_OK;
  REQUIRE(P && Pt, TMOE_E_ARG, "null pointer");
  REQUIRE(aligned16(Pt), TMOE_E_ALIGN, "Pt not 16-byte aligned");
  return launch_repack_tiled((hipStream_t)stream, P, R, K, ldp, Pt);
}

int tmoe_unpack_tiled(void *stream, const uint8_t *Pt, int64_t R, int64_t K, int8_t *T) {
  clear_error();
  REQUIRE(R >= 0 && K >= 0, TMOE_E_ARG, "negative size");
  if (R == 0 || K == 0) return TMOE_OK;
  REQUIRE(Pt && T, TMOE_E_ARG, "null pointer");
  REQUIRE(aligned16(Pt), TMOE_E_ALIGN, "Pt not 16-byte aligned");
  return launch_unpack_tiled((hipStream_t)stream, Pt, R, K, T);
}

// ------------------------------------------------------------ ternary linear
size_t tmoe_linear_workspace_bytes(int64_t T, int64_t K) {
  if (T <= 0 || K <= 0) return 0;
  return linear_ws_bytes(T, K);
}

int tmoe_ternary_linear(void *stream, const uint8_t *Pt, const float *s, int64_t N, int64_t K, const uint16_t *X,
                        int64_t ldx, int64_t T, float *Y, int64_t ldy, void *ws, size_t ws_bytes) {
  clear_error();
  REQUIRE(N >= 0 && K >= 0 && T >= 0, TMOE_E_ARG, "negative size");
  if (N == 0 || T == 0) return TMOE_OK;
  REQUIRE(K > 0, TMOE_E_SHAPE, "K must be positive");
  REQUIRE(ldx >= K && ldy >= N, TMOE_E_SHAPE, "ldx < K or ldy < N");
  REQUIRE(Pt && s && X && Y, TMOE_E_ARG, "null pointer");
  REQUIRE(aligned16(Pt), TMOE_E_ALIGN, "Pt not 16-byte aligned");
  REQUIRE(aligned4(s) && aligned4(Y) && ((uintptr_t)X & 1) == 0, TMOE_E_ALIGN, "misaligned s, X or Y");
  size_t need = linear_ws_bytes(T, K);
  REQUIRE(need == 0 || (ws && ws_bytes >= need && aligned16(ws)), TMOE_E_WORKSPACE,
          "workspace needs %zu bytes (16-aligned)", need);
  return launch_linear((hipStream_t)stream, Pt, s, N, K, X, ldx, T, Y, ldy, ws);
}

size_t tmoe_linear_packed_workspace_bytes(int64_t N, int64_t K, int64_t T) {
  if (N <= 0 || K <= 0) return 0;
  return align_up((size_t)tmoe_tiled_bytes(N, K), 256) + tmoe_linear_workspace_bytes(T, K);
}

int tmoe_ternary_linear_packed(void *stream, const uint8_t *P, int64_t ldp, const float *s, int64_t N, int64_t K,
                               const uint16_t *X, int64_t ldx, int64_t T, float *Y, int64_t ldy, void *ws,
                               size_t ws_bytes) {
  clear_error();
  REQUIRE(N >= 0 && K >= 0 && T >= 0, TMOE_E_ARG, "negative size");
  if (N == 0 || T == 0) return TMOE_OK;
  REQUIRE(K > 0, TMOE_E_SHAPE, "K must be positive");
  REQUIRE(ldp >= (K + 4) / 5, TMOE_E_SHAPE, "ldp < ceil(K/5)");
  REQUIRE(ldx >= K && ldy >= N, TMOE_E_SHAPE, "ldx < K or ldy < N");
  REQUIRE(P && s && X && Y, TMOE_E_ARG, "null pointer");
  const size_t need = tmoe_linear_packed_workspace_bytes(N, K, T);
  REQUIRE(ws && ws_bytes >= need && aligned16(ws), TMOE_E_WORKSPACE, "workspace needs %zu bytes (16-aligned)", need);
  uint8_t *Pt = static_cast<uint8_t *>(ws);
  const size_t tiled = align_up((size_t)tmoe_tiled_bytes(N, K), 256);
  int rc = tmoe_repack_tiled(stream, P, N, K, ldp, Pt);
  if (rc) return rc;
  return tmoe_ternary_linear(stream, Pt, s, N, K, X, ldx, T, Y, ldy, static_cast<char *>(ws) + tiled, ws_bytes - tiled);
}

// -------------------------------------------------------------------- router
size_t tmoe_router_workspace_bytes(int64_t T, int64_t E) {
  if (T < 0 || E <= 0) return 0;
  return router_ws_bytes(T, E, kRouterMaxH);
}

static int check_router(const uint16_t *X, int64_t T, int64_t H, const float *Wr, int64_t E, int k, int32_t *idx,
                        float *w) {
  REQUIRE(T >= 0 && H > 0 && E > 0, TMOE_E_ARG, "bad sizes T=%lld H=%lld E=%lld", (long long)T, (long long)H,
          (long long)E);
  REQUIRE(k >= 1 && k <= 16 && k <= E, TMOE_E_SHAPE, "need 1 <= k <= min(E, 16), k=%d", k);
  REQUIRE(E <= 1024, TMOE_E_UNSUPPORTED, "E=%lld > 1024", (long long)E);
  REQUIRE(H % 8 == 0 && H <= 8192, TMOE_E_UNSUPPORTED, "H must be a multiple of 8 and <= 8192");
  if (T == 0) return TMOE_OK;
  REQUIRE(X && Wr && idx && w, TMOE_E_ARG, "null pointer");
  REQUIRE(aligned16(X) && aligned16(Wr) && aligned4(idx) && aligned4(w), TMOE_E_ALIGN, "misaligned pointer");
  return TMOE_OK;
}

int tmoe_router_topk(void *stream, const uint16_t *X, int64_t T, int64_t H, const float *Wr, const float *bias,
                     int64_t E, int k, int32_t *idx, float *w, float *logits, int32_t *n_fixup, void *ws,
                     size_t ws_bytes) {
  clear_error();
  int rc = check_router(X, T, H, Wr, E, k, idx, w);
  if (rc) return rc;
  if (T == 0) return TMOE_OK;
  size_t need = router_ws_bytes(T, E, kRouterMaxH);
  REQUIRE(ws && ws_bytes >= need && aligned16(ws), TMOE_E_WORKSPACE, "workspace needs %zu bytes", need);
  return launch_router((hipStream_t)stream, X, T, H, Wr, bias, E, k, idx, w, logits, n_fixup,
                       router_ws_carve(ws, T, E, kRouterMaxH));
}

// ------------------------------------------------------------ attention half
static int check_attn(const tmoe_attn_weights *W) {
  REQUIRE(W, TMOE_E_ARG, "null weights");
  REQUIRE(W->reserved == 0, TMOE_E_ARG, "reserved must be 0");
  REQUIRE(W->hidden == 2048 && W->head_dim == 128 && (int64_t)W->n_heads * W->head_dim == W->hidden &&
              W->n_kv_heads > 0 && W->n_heads == 4 * W->n_kv_heads,
          TMOE_E_UNSUPPORTED, "attention: hidden 2048, head_dim 128, n_heads = hidden / 128 = 4 n_kv_heads");
  REQUIRE(W->window >= 0 && W->rotary_dim >= 0 && W->rotary_dim <= W->head_dim && W->rotary_dim % 2 == 0,
          TMOE_E_SHAPE, "bad window or rotary_dim");
  REQUIRE(!(W->window > 0 && W->rotary_dim > 0) || W->rope_base > 1.0, TMOE_E_ARG, "rope_base must be > 1");
  REQUIRE(W->qkv_p && W->qkv_s && W->o_p && W->o_s, TMOE_E_ARG, "null weight pointer");
  REQUIRE(aligned16(W->qkv_p) && aligned16(W->o_p) && aligned16(W->qkv_s) && aligned16(W->o_s), TMOE_E_ALIGN,
          "misaligned weights");
  return TMOE_OK;
}

size_t tmoe_attention_workspace_bytes(int64_t T, const tmoe_attn_weights *W) {
  if (T < 0 || check_attn(W) != TMOE_OK) return 0;
  return attn_ws_bytes(T > 0 ? T : 1, W->n_heads, W->n_kv_heads, W->head_dim);
}

int tmoe_attention_forward(void *stream, const tmoe_attn_weights *W, const uint16_t *X, int64_t T, int64_t pos0,
                           float *k_cache, float *v_cache, int64_t cache_cap, float *O, uint16_t *X_out, void *ws,
                           size_t ws_bytes) {
  clear_error();
  int rc = check_attn(W);
  if (rc) return rc;
  REQUIRE(T >= 0 && pos0 >= 0 && cache_cap > 0, TMOE_E_ARG, "bad T, pos0 or cache_cap");
  if (T == 0) return TMOE_OK;
  REQUIRE(T <= (1 << 24) && pos0 <= ((int64_t)1 << 40), TMOE_E_UNSUPPORTED, "T or pos0 too large");
  REQUIRE(X && k_cache && v_cache && (O || X_out), TMOE_E_ARG, "null X, cache, or neither O nor X_out");
  REQUIRE(aligned16(X) && aligned16(k_cache) && aligned16(v_cache) && (!O || aligned16(O)) &&
              (!X_out || aligned16(X_out)),
          TMOE_E_ALIGN, "misaligned pointer");
  if (W->window > 0)
    REQUIRE(cache_cap >= W->window + T - 1, TMOE_E_SHAPE, "sliding cache needs capacity >= window + T - 1");
  else
    REQUIRE(cache_cap >= pos0 + T, TMOE_E_SHAPE, "global cache needs capacity >= pos0 + T");
  const size_t need = attn_ws_bytes(T, W->n_heads, W->n_kv_heads, W->head_dim);
  REQUIRE(ws && ws_bytes >= need && aligned16(ws), TMOE_E_WORKSPACE, "workspace needs %zu bytes", need);
  return launch_attention((hipStream_t)stream, *W, X, T, pos0, k_cache, v_cache, cache_cap, O, X_out, ws);
}

// ------------------------------------------------------ host-resident experts
int tmoe_host_alloc(size_t bytes, void **host, void **device) {
  clear_error();
  REQUIRE(bytes > 0 && host && device, TMOE_E_ARG, "need bytes > 0 and both outputs");
  *host = *device = nullptr;
  void *h = nullptr;
  hipError_t e = hipHostMalloc(&h, bytes, hipHostMallocMapped | hipHostMallocNonCoherent);
  if (e != hipSuccess) return hip_fail(e, "hipHostMalloc");
  void *d = nullptr;
  e = hipHostGetDevicePointer(&d, h, 0);
  if (e != hipSuccess || !d) {
    (void)hipHostFree(h);
    return hip_fail(e != hipSuccess ? e : hipErrorInvalidValue, "hipHostGetDevicePointer");
  }
  *host = h;
  *device = d;
  return TMOE_OK;
}

int tmoe_host_free(void *host) {
  clear_error();
  if (!host) return TMOE_OK;
  hipError_t e = hipHostFree(host);
  return e == hipSuccess ? TMOE_OK : hip_fail(e, "hipHostFree");
}

// ------------------------------------------------------------------- LM head
size_t tmoe_lm_head_workspace_bytes(int64_t T, int64_t V, int k) {
  if (T <= 0 || V <= 0 || k <= 0 || V > (int64_t)1 << 31) return 0;
  return lmh_ws_bytes(T, V, k);
}

int tmoe_lm_head_topk(void *stream, const uint16_t *X, int64_t T, int64_t H, const uint16_t *W, int64_t V, int k,
                      int32_t *idx, float *val, float *logits, int32_t *n_fixup, void *ws, size_t ws_bytes) {
  clear_error();
  REQUIRE(T >= 0 && H > 0 && V > 0 && k >= 1, TMOE_E_ARG, "bad sizes");
  if (T == 0) return TMOE_OK;
  REQUIRE(X && W && idx && val, TMOE_E_ARG, "null pointer");
  REQUIRE(T == 1 || T == 2 || T == 4, TMOE_E_UNSUPPORTED, "lm head: T must be 1, 2 or 4");
  REQUIRE(H == 512 || H == 1024 || H == 2048 || H == 4096, TMOE_E_UNSUPPORTED,
          "lm head: hidden must be 512, 1024, 2048 or 4096");
  REQUIRE(k <= 16, TMOE_E_UNSUPPORTED, "lm head: k <= 16");
  REQUIRE(k < V, TMOE_E_SHAPE, "lm head: need k < V");
  REQUIRE(V <= ((int64_t)1 << 20), TMOE_E_UNSUPPORTED, "lm head: V <= 2^20");
  REQUIRE(aligned16(X) && aligned16(W) && aligned4(idx) && aligned4(val) && (!logits || aligned4(logits)) &&
              (!n_fixup || aligned4(n_fixup)),
          TMOE_E_ALIGN, "misaligned pointer");
  const size_t need = lmh_ws_bytes(T, V, k);
  REQUIRE(ws && ws_bytes >= need && aligned16(ws), TMOE_E_WORKSPACE, "workspace needs %zu bytes", need);
  return launch_lm_head((hipStream_t)stream, X, T, H, W, V, k, idx, val, logits, n_fixup, ws);
}

// ------------------------------------------------------------------ grouping
size_t tmoe_group_workspace_bytes(int64_t T, int k, int64_t E) {
  if (T < 0 || k <= 0 || E <= 0) return 0;
  return group_ws_bytes(T, k, E);
}

int tmoe_group_by_expert(void *stream, const int32_t *idx, int64_t T, int k, int64_t E, int32_t *counts,
                         int32_t *offsets, int32_t *sorted_token, int32_t *sorted_slot, int32_t *pos, void *ws,
                         size_t ws_bytes) {
  clear_error();
  REQUIRE(T >= 0 && E > 0 && k >= 1, TMOE_E_ARG, "bad sizes");
  REQUIRE(k <= 64 && k <= E, TMOE_E_SHAPE, "k must be <= min(E, 64)");
  REQUIRE(E <= 1024, TMOE_E_UNSUPPORTED, "E > 1024");
  REQUIRE(T * k < (int64_t)1 << 30, TMOE_E_UNSUPPORTED, "T*k too large");
  REQUIRE(counts && offsets, TMOE_E_ARG, "null counts/offsets");
  if (T > 0) REQUIRE(idx && sorted_token && sorted_slot && pos, TMOE_E_ARG, "null pointer");
  size_t need = group_ws_bytes(T, k, E);
  REQUIRE(need == 0 || (ws && ws_bytes >= need && aligned16(ws)), TMOE_E_WORKSPACE, "workspace needs %zu bytes",
          need);
  return launch_group((hipStream_t)stream, idx, T, k, E, counts, offsets, sorted_token, sorted_slot, pos,
                      group_ws_carve(ws, T, k, E), nullptr, nullptr, 16);
}

// --------------------------------------------------------------- expert FFN
static int check_weights(const tmoe_moe_weights *W) {
  REQUIRE(W, TMOE_E_ARG, "null weights");
  REQUIRE(W->reserved == 0, TMOE_E_ARG, "reserved field must be 0");
  REQUIRE(W->hidden > 0 && W->inter > 0 && W->n_experts > 0, TMOE_E_ARG, "bad layer sizes");
  REQUIRE(W->top_k >= 1 && W->top_k <= 16 && W->top_k <= W->n_experts, TMOE_E_SHAPE, "bad top_k");
  REQUIRE(W->n_experts <= 1024, TMOE_E_UNSUPPORTED, "n_experts > 1024");
  REQUIRE(W->hidden % 64 == 0 && W->inter % 64 == 0, TMOE_E_UNSUPPORTED, "hidden and inter must be multiples of 64");
  REQUIRE(W->hidden <= 8192 && W->inter <= 8192, TMOE_E_UNSUPPORTED, "hidden/inter > 8192");
  REQUIRE(W->gate_p && W->up_p && W->down_p && W->gate_s && W->up_s && W->down_s, TMOE_E_ARG, "null expert weights");
  REQUIRE(aligned16(W->gate_p) && aligned16(W->up_p) && aligned16(W->down_p), TMOE_E_ALIGN, "weights misaligned");
  REQUIRE(aligned16(W->gate_s) && aligned16(W->up_s) && aligned16(W->down_s), TMOE_E_ALIGN, "scales misaligned");
  REQUIRE(W->stride_gu >= tmoe_tiled_bytes(W->inter, W->hidden) && W->stride_gu % 16 == 0, TMOE_E_SHAPE,
          "stride_gu too small or not a multiple of 16");
  REQUIRE(W->stride_d >= tmoe_tiled_bytes(W->hidden, W->inter) && W->stride_d % 16 == 0, TMOE_E_SHAPE,
          "stride_d too small or not a multiple of 16");
  return TMOE_OK;
}

size_t tmoe_ffn_workspace_bytes(int64_t T, const tmoe_moe_weights *W) {
  if (T < 0 || !W || check_weights(W)) return 0;
  return ffn_ws_bytes(T, W->top_k, W->n_experts, W->hidden, W->inter);
}

int tmoe_expert_ffn(void *stream, const tmoe_moe_weights *W, const uint16_t *X, int64_t T, const int32_t *offsets,
                    const int32_t *sorted_token, float clamp, float *O, float *Hout, void *ws, size_t ws_bytes) {
  clear_error();
  int rc = check_weights(W);
  if (rc) return rc;
  REQUIRE(T >= 0, TMOE_E_ARG, "negative T");
  REQUIRE(!(clamp != clamp) && clamp >= 0, TMOE_E_ARG, "clamp must be >= 0 (INFINITY disables)");
  if (T == 0) return TMOE_OK;
  REQUIRE(X && offsets && sorted_token && O, TMOE_E_ARG, "null pointer");
  REQUIRE(aligned16(X) && aligned16(O) && (!Hout || aligned16(Hout)), TMOE_E_ALIGN, "misaligned X, O or Hout");
  size_t need = ffn_ws_bytes(T, W->top_k, W->n_experts, W->hidden, W->inter);
  REQUIRE(ws && ws_bytes >= need && aligned16(ws), TMOE_E_WORKSPACE, "workspace needs %zu bytes", need);
  return launch_ffn((hipStream_t)stream, W, X, T, offsets, sorted_token, clamp, O, Hout,
                    ffn_ws_carve(ws, T, W->top_k, W->n_experts, W->hidden, W->inter), false);
}

// ------------------------------------------------------------------ combine
int tmoe_combine(void *stream, const float *O, const float *w, const int32_t *pos, int64_t T, int k, int64_t H,
                 float *Y, const uint16_t *resid_in, uint16_t *resid_out) {
  clear_error();
  REQUIRE(T >= 0 && k >= 1 && k <= 64 && H > 0, TMOE_E_ARG, "bad sizes");
  REQUIRE(H % 8 == 0, TMOE_E_UNSUPPORTED, "H must be a multiple of 8");
  if (T == 0) return TMOE_OK;
  REQUIRE(O && w && pos && (Y || resid_out), TMOE_E_ARG, "null pointer");
  REQUIRE(!resid_out || resid_in, TMOE_E_ARG, "resid_out needs resid_in");
  REQUIRE(aligned16(O) && (!Y || aligned16(Y)) && (!resid_in || aligned16(resid_in)) &&
              (!resid_out || aligned16(resid_out)),
          TMOE_E_ALIGN, "misaligned pointer");
  return launch_combine((hipStream_t)stream, O, w, pos, T, k, H, Y, resid_in, resid_out);
}

// -------------------------------------------------------------- whole layer
struct LayerWs {
  size_t router, group, ffn, total;
  size_t off_router, off_group, off_ffn, off_idx, off_w, off_pos, off_counts, off_offsets, off_st, off_ss, off_O;
};

static LayerWs layer_ws(int64_t T, const tmoe_moe_weights *W) {
  LayerWs L{};
  const int64_t E = W->n_experts, k = W->top_k, H = W->hidden, P = T * k;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.router = router_ws_bytes(T, E, H);
  L.group = group_ws_bytes(T, (int)k, E);
  L.ffn = ffn_ws_bytes(T, (int)k, E, H, W->inter);
  L.off_router = take(L.router);
  L.off_group = take(L.group);
  L.off_ffn = take(L.ffn);
  L.off_idx = take(P * 4);
  L.off_w = take(P * 4);
  L.off_pos = take(P * 4);
  L.off_counts = take(E * 4);
  L.off_offsets = take((E + 1) * 4);
  L.off_st = take(P * 4);
  L.off_ss = take(P * 4);
  // expert outputs; the decode path with few pairs fuses the combine and needs none
  L.off_O = take(T <= kDecodePathMaxT && P <= kDcMaxPairs ? 0 : (size_t)P * H * 4);
  L.total = o;
  return L;
}

int tmoe_moe_workspace_bytes(int64_t T, const tmoe_moe_weights *W, size_t *out) {
  clear_error();
  REQUIRE(out, TMOE_E_ARG, "null out");
  REQUIRE(T >= 0, TMOE_E_ARG, "negative T");
  int rc = check_weights(W);
  if (rc) return rc;
  *out = layer_ws(T, W).total;
  return TMOE_OK;
}

int tmoe_moe_forward(void *stream, const tmoe_moe_weights *W, const uint16_t *X, int64_t T, float *Y,
                     const tmoe_moe_options *opt, void *ws, size_t ws_bytes) {
  clear_error();
  return moe_forward_impl(stream, W, X, T, Y, opt, ws, ws_bytes);
}

}  // extern "C"

namespace tmoe {

int moe_workspace_total(int64_t T, const tmoe_moe_weights *W, size_t *out) {
  int rc = check_weights(W);
  if (rc) return rc;
  REQUIRE(T >= 0, TMOE_E_ARG, "negative T");
  *out = layer_ws(T, W).total;
  return TMOE_OK;
}

int moe_forward_impl(void *stream, const tmoe_moe_weights *W, const uint16_t *X, int64_t T, float *Y,
                     const tmoe_moe_options *opt, void *ws, size_t ws_bytes) {
  int rc = check_weights(W);
  if (rc) return rc;
  REQUIRE(T >= 0, TMOE_E_ARG, "negative T");
  tmoe_moe_options o{};
  o.clamp = 7.0f;
  if (opt) o = *opt;
  REQUIRE(o.reserved0 == 0, TMOE_E_ARG, "reserved option must be 0");
  REQUIRE(!(o.clamp != o.clamp) && o.clamp >= 0, TMOE_E_ARG, "clamp must be >= 0");
  if (T == 0) return TMOE_OK;
  REQUIRE(X && (Y || o.resid_out), TMOE_E_ARG, "null X, or neither Y nor resid_out");
  REQUIRE(W->router_w, TMOE_E_ARG, "null router weights");
  REQUIRE(aligned16(X) && (!Y || aligned16(Y)) && aligned16(W->router_w) &&
              (!o.resid_out || aligned16(o.resid_out)),
          TMOE_E_ALIGN, "misaligned pointer");
  LayerWs L = layer_ws(T, W);
  REQUIRE(ws && ws_bytes >= L.total && aligned16(ws), TMOE_E_WORKSPACE, "workspace needs %zu bytes", L.total);
  hipStream_t st = (hipStream_t)stream;
  char *base = (char *)ws;
  const int64_t E = W->n_experts, H = W->hidden;
  const int k = W->top_k;
  int32_t *idx = o.idx ? o.idx : (int32_t *)(base + L.off_idx);
  float *wt = o.w ? o.w : (float *)(base + L.off_w);
  int32_t *pos = o.pos ? o.pos : (int32_t *)(base + L.off_pos);
  int32_t *counts = (int32_t *)(base + L.off_counts);
  int32_t *offsets = (int32_t *)(base + L.off_offsets);
  int32_t *st_tok = (int32_t *)(base + L.off_st);
  int32_t *st_slot = (int32_t *)(base + L.off_ss);
  float *O = (float *)(base + L.off_O);
  const RouterWs rw = router_ws_carve(base + L.off_router, T, E, H);
  const FfnWs fw = ffn_ws_carve(base + L.off_ffn, T, k, E, H, W->inter);
  if (T <= kDecodePathMaxT) {
    // logits; gate/up with the certified top-k and grouping in its prologue; down + combine
    int depth = 0, nb = 0;
    rc = launch_router_logits(st, X, T, H, W->router_w, W->router_bias, E, rw, &depth, &nb);
    if (rc) return rc;
    const DecodeRoute r{rw.lg, rw.bnd, depth, nb, topk_bound_scale(depth), W->router_w, W->router_bias, idx,
                        o.n_fixup, st_tok, st_slot, pos, wt, nullptr, nullptr, nullptr};
    return launch_decode_tail(st, W, X, T, o.clamp, r, fw, O, Y, o.resid_out ? X : nullptr, o.resid_out);
  }
  rc = launch_router(st, X, T, H, W->router_w, W->router_bias, E, k, idx, wt, nullptr, o.n_fixup, rw);
  if (rc) return rc;
  // the grouping also writes the work tiles of the expert kernels' form
  const bool blocked = ffn_blocked(T * k, E, H, W->inter);
  rc = launch_group(st, idx, T, k, E, counts, offsets, st_tok, st_slot, pos, group_ws_carve(base + L.off_group, T, k, E),
                    blocked ? fw.blocks : fw.tiles, blocked ? fw.nblocks : fw.ntiles, blocked ? 64 : 16);
  if (rc) return rc;
  rc = launch_ffn(st, W, X, T, offsets, st_tok, o.clamp, O, nullptr, fw, true);
  if (rc) return rc;
  return launch_combine(st, O, wt, pos, T, k, H, Y, o.resid_out ? X : nullptr, o.resid_out);
}

}  // namespace tmoe

extern "C" {

int tmoe_profile_begin(int kernel, int capacity) {
  clear_error();
  REQUIRE(kernel >= TMOE_KERNEL_ROUTER_LOGITS && kernel <= TMOE_KERNEL_ATTENTION, TMOE_E_ARG, "unknown kernel id %d",
          kernel);
  REQUIRE(capacity > 0 && capacity <= (1 << 20), TMOE_E_ARG, "capacity out of range");
  REQUIRE(g_prof.kernel == 0, TMOE_E_ARG, "a profiling window is already open");
  g_prof.start = new hipEvent_t[capacity]();
  g_prof.stop = new hipEvent_t[capacity]();
  g_prof.cap = capacity;
  for (int i = 0; i < capacity; ++i) {
    // timing-only events: no system-scope fence (no cache write-back around the kernel)
    hipError_t e = hipEventCreateWithFlags(&g_prof.start[i], hipEventDisableSystemFence);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&g_prof.stop[i], hipEventDisableSystemFence);
    if (e != hipSuccess) {
      prof_free();
      return hip_fail(e, "hipEventCreate");
    }
  }
  g_prof.kernel = kernel;
  g_prof.n = 0;
  return TMOE_OK;
}

int tmoe_profile_end(float *ms, int capacity, int *count) {
  clear_error();
  REQUIRE(count && (ms || capacity == 0), TMOE_E_ARG, "null output");
  REQUIRE(g_prof.kernel != 0, TMOE_E_ARG, "no profiling window open");
  int n = g_prof.n < capacity ? g_prof.n : capacity;
  int rc = TMOE_OK;
  for (int i = 0; i < n && rc == TMOE_OK; ++i) {
    hipError_t e = hipEventSynchronize(g_prof.stop[i]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms[i], g_prof.start[i], g_prof.stop[i]);
    if (e != hipSuccess) rc = hip_fail(e, "profile events");
  }
  *count = n;
  prof_free();
  return rc;
}

}  // extern "C"
