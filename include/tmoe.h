/*
 * tmoe.h - C ABI of the ternary Mixture-of-Experts expert layer for AMD
 * Instinct MI355X (gfx950).
 *
 * What the layer computes (the pages are the authority):
 *  - Weights are ternary, {-1, 0, +1} times one fp32 scale per output row
 *    (ai.thesatyajit.com, "Maple-Preview: a 20B reasoning model where 97% of
 *    the weights are -1, 0, or +1", section "The claim, verified from the
 *    bytes"); a ternary weight skips, adds or subtracts its activation
 *    (codeinsider.com.br, section "Pesos ternarios").
 *  - Five trits are packed into one byte, 3^5 = 243 <= 256 (ai.thesatyajit.com,
 *    section "The 5.31 GB claim reconciles").
 *  - The router stays full precision and picks 8 of 256 experts per token
 *    (ai.thesatyajit.com, "The claim, verified from the bytes";
 *    codeinsider.com.br, "256 experts, 8 ativos").
 *  - One expert maps a token x to o = Wd h, where h = SiLU(min(g, 7)) times
 *    the clip of u to [-7, 7], g = Wg x and u = Wu x (ai.thesatyajit.com,
 *    "The shipped code does no quantization").
 *  - Shapes: hidden 2048, 256 experts, top 8, moe_intermediate_size 512
 *    (jj-blog Maple-Preview news, architecture list).
 *
 * Conventions (all functions):
 *  - Return an int status: TMOE_OK (0) or a negative TMOE_E_* code. The library
 *    never aborts, prints or exits. tmoe_last_error() gives a thread-local
 *    message for the last failure on the calling thread.
 *  - The caller owns every buffer. Device functions never allocate; scratch
 *    memory comes from a caller workspace of the size the matching
 *    *_workspace_bytes query returns.
 *  - Device functions are asynchronous on the caller's HIP stream, passed as
 *    `void *stream` (a hipStream_t; NULL means the default stream).
 *    Arguments are checked synchronously before anything is enqueued; a
 *    failed check enqueues nothing. A HIP launch error returns TMOE_E_HIP.
 *  - Sizes are int64_t. Device pointers must be 16-byte aligned unless stated
 *    otherwise (TMOE_E_ALIGN).
 *  - Matrices are row-major. A weight matrix is [rows = outputs][cols = inputs]
 *    (the F.linear orientation of the printed forward).
 *  - Packed bytes given to device kernels must be valid codes (<= 242); check
 *    untrusted bytes with tmoe_validate_packed_host first.
 *  - bf16 values are passed as uint16_t bit patterns.
 */
#ifndef TMOE_H
#define TMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ----------------------------------------------------------------- status */
enum {
  TMOE_OK = 0,
  TMOE_E_ARG = -1,         /* null pointer, negative size, bad enum value */
  TMOE_E_SHAPE = -2,       /* inconsistent or unsupported dimensions */
  TMOE_E_ALIGN = -3,       /* device pointer not 16-byte aligned */
  TMOE_E_BADPACK = -4,     /* a packed byte > 242 (not a 5-trit code) */
  TMOE_E_WORKSPACE = -5,   /* workspace null or smaller than required */
  TMOE_E_UNSUPPORTED = -6, /* valid request this library does not implement */
  TMOE_E_HIP = -7          /* the HIP runtime reported an error */
};

/* Static string naming a status code ("TMOE_OK", "TMOE_E_ARG", ...). */
const char *tmoe_status_str(int status);
/* Message describing the last failure on this thread ("" if none). */
const char *tmoe_last_error(void);
/* ABI version: major * 10000 + minor * 100 + patch. */
int tmoe_version(void);

/* -------------------------------------------------- host weight preparation
 * Offline steps (not on the timed path). Host pointers, synchronous.
 */

/* Absmean ternarization of fp32 W [R][K] (ai.thesatyajit.com, "The claim,
 * verified from the bytes": {-s, 0, +s} per row, absmean, per-output-channel
 * scale).
 *   s[r] = fp32( (sum_i |W[r][i]|) / K ), the sum taken in fp64 in index order;
 *   T[r][i] = sign(W[r][i]) if 2|W[r][i]| > s[r], else 0 (ties go to 0; an
 *   all-zero row gives s = 0 and zero trits).
 * W must be finite (TMOE_E_ARG otherwise, nothing written).
 * Out: T int8 [R][K], s fp32 [R]. */
int tmoe_ternarize_absmean_host(const float *W, int64_t R, int64_t K, int8_t *T, float *s);

/* Canonical packing (ai.thesatyajit.com, "The 5.31 GB claim reconciles"):
 * byte j of row r is sum_{q<5} (T[r][5j+q] + 1) * 3^q, trits past K count as
 * 0. P is uint8 [R][ldp], ldp >= ceil(K/5); bytes [ceil(K/5), ldp) of each row
 * are not written. T values outside {-1,0,1} give TMOE_E_ARG. */
int tmoe_pack_host(const int8_t *T, int64_t R, int64_t K, uint8_t *P, int64_t ldp);

/* Inverse of tmoe_pack_host: T[r][5j+q] = ((P[r][j] / 3^q) mod 3) - 1 for
 * 5j+q < K. A byte > 242 gives TMOE_E_BADPACK (T then partly written). */
int tmoe_unpack_host(const uint8_t *P, int64_t R, int64_t K, int64_t ldp, int8_t *T);

/* Counts bytes > 242 among the ceil(K/5) data bytes of each row into *n_bad;
 * returns TMOE_E_BADPACK if any, TMOE_OK otherwise. */
int tmoe_validate_packed_host(const uint8_t *P, int64_t R, int64_t K, int64_t ldp, int64_t *n_bad);

/* ----------------------------------------------------- device weight layout
 * The GEMM kernels read weights in a "tiled" layout holding the same trits,
 * still 5 per byte in base 3 (digit = trit + 1), but re-ordered for the MFMA:
 * rows are grouped in tiles of 16 (the MFMA row block); a row's input indices
 * are split into four quarters of 5Q indices (Q = ceil(ceil(K/5)/4) rounded up
 * to even), quarter g of row i being read by lane i + 16g, so that each 64-lane
 * wavefront load is one contiguous run. Within a quarter, bytes come in steps
 * of 8 (and a last, shorter step of Q mod 8 bytes): byte 2p + h of a step
 * holds, as digit q, the trit of quarter input index 40*step + 10p + 2q + h,
 * so the 8 trits one MFMA lane needs cover 8 consecutive input indices.
 * Indices past K, and rows past R, hold zero trits. The tiled form is
 * lossless: tmoe_unpack_tiled returns the same trits as the canonical bytes.
 * Size in bytes: tmoe_tiled_bytes(R, K) = ceil(R/16) * 16 * 4 * Q.
 */
int64_t tmoe_tiled_bytes(int64_t R, int64_t K);

/* Device absmean ternarize + canonical pack of fp32 W [R][K] (row stride K):
 * the definition of tmoe_ternarize_absmean_host, bit for bit for any finite
 * fp32 input (the fp64 sum of |w| runs in index order, one thread per row).
 * Out: P [R][ldp] (bytes past ceil(K/5) untouched), s [R]. Non-finite inputs
 * are not checked on the device. */
int tmoe_ternarize_pack(void *stream, const float *W, int64_t R, int64_t K, uint8_t *P, int64_t ldp, float *s);

/* Device unpack of canonical bytes (the bit-exact parity hook): T int8 [R][K]. */
int tmoe_unpack(void *stream, const uint8_t *P, int64_t R, int64_t K, int64_t ldp, int8_t *T);

/* Canonical P [R][ldp] -> tiled Pt [tmoe_tiled_bytes(R, K)]. */
int tmoe_repack_tiled(void *stream, const uint8_t *P, int64_t R, int64_t K, int64_t ldp, uint8_t *Pt);

/* Tiled Pt -> trits int8 [R][K] (parity hook for the tiled layout). */
int tmoe_unpack_tiled(void *stream, const uint8_t *Pt, int64_t R, int64_t K, int8_t *T);

/* ------------------------------------------------- synthetic weight source
 * Counter-based generator (not part of the layer; it draws the synthetic
 * weights in HBM). out[i] = IH12(Philox4x64-10(counter = (first + i, stream_id,
 * 0, 0), key = (key0, key1))) where IH12 sums the twelve little-endian 16-bit
 * halves of output words 0..2, subtracts 393210 and scales by 2^-16; then
 * out[i] *= mult (one fp32 multiply; mult = 1 leaves it exact).
 * Philox: Salmon et al., "Parallel random numbers: as easy as 1, 2, 3" (SC'11).
 */
int tmoe_synth_ih12(void *stream, uint64_t key0, uint64_t key1, uint64_t stream_id, uint64_t first, int64_t n,
                    float mult, float *out);

/* ------------------------------------------------------------ ternary linear
 * Y[n][o] = s[o] * sum_i T[o][i] * X[n][i] for n < T tokens, o < N outputs
 * (codeinsider.com.br, "Pesos ternarios": add / subtract / skip; the dense
 * definition with dequantized weights). fp32 accumulation.
 *   Pt: tiled packed weights of an [N][K] matrix; s: fp32 [N];
 *   X: bf16 [T][ldx] (ldx >= K, element stride; 2-byte alignment suffices);
 *   Y: fp32 [T][ldy] (ldy >= N).
 * ws: workspace of tmoe_linear_workspace_bytes(T, K) bytes; the current
 *   kernels need none (0 bytes, ws may be NULL).
 * Very tall operands with few tokens (K = 2048, T <= 16, N >= 131,072 rows,
 * contiguous 16-byte-aligned X) take a streaming kernel whose wavefronts walk
 * row tiles with the next tile's weights in flight; the result is the same
 * up to fp32 summation order. Errors: TMOE_E_UNSUPPORTED when T > 16 and
 * N > 4,194,240 rows (more than 65,535 groups of four row tiles). */
size_t tmoe_linear_workspace_bytes(int64_t T, int64_t K);
int tmoe_ternary_linear(void *stream, const uint8_t *Pt, const float *s, int64_t N, int64_t K, const uint16_t *X,
                        int64_t ldx, int64_t T, float *Y, int64_t ldy, void *ws, size_t ws_bytes);

/* The same product from canonical packed bytes: P uint8 [N][ldp], ldp >=
 * ceil(K/5), row-major, 5 trits per byte as tmoe_pack_host writes them
 * (ai.thesatyajit.com, "The 5.31 GB claim reconciles": five base-3 digits per
 * byte). The call first writes the tiled image of P into the workspace
 * (tmoe_repack_tiled), then runs tmoe_ternary_linear on it, both on `stream`;
 * Y is the same as tmoe_ternary_linear's on that image. ws: at least
 * tmoe_linear_packed_workspace_bytes(N, K, T) bytes, 16-byte aligned, owned
 * by the caller and free for reuse when the stream has passed the call. A
 * caller that multiplies the same weights many times repacks once and calls
 * tmoe_ternary_linear. Errors: as tmoe_repack_tiled and tmoe_ternary_linear;
 * TMOE_E_WORKSPACE when ws is short. */
size_t tmoe_linear_packed_workspace_bytes(int64_t N, int64_t K, int64_t T);
int tmoe_ternary_linear_packed(void *stream, const uint8_t *P, int64_t ldp, const float *s, int64_t N, int64_t K,
                               const uint16_t *X, int64_t ldx, int64_t T, float *Y, int64_t ldy, void *ws,
                               size_t ws_bytes);

/* ------------------------------------------------------------------ router
 * Full-precision router (ai.thesatyajit.com, "The claim, verified from the
 * bytes": routers stay sharp; 8 of 256 chosen by logit margins).
 *   logits[t][e] = sum_i X[t][i] * Wr[e][i] + bias[e]   (bias may be NULL)
 *   idx[t][0..k)  = the k largest logits, descending, equal logits -> lower e
 *   w[t][j]       = softmax over the k selected logits
 * The top-k is certified: logits are accumulated in fp64 from exact
 * products and carry a rigorous rounding-error bound; a token whose
 * top-(k+1) ranking is not separated by that bound is recomputed in
 * double-double arithmetic on the device. Indices therefore equal those of
 * the exact logits except for logits closer than ~1e-30 relative.
 * From 1024 tokens on, when `logits` is NULL, the logits are first formed on the
 * bf16 matrix cores (each fp32 weight as the sum of two bf16 parts, with a
 * rigorous bound, about 2.5e-5 of |x| |w_e| for H = 2048) only to pick
 * each token's candidates (the k+1 largest and every expert within twice
 * that bound of the (k+1)-th); the candidates are recomputed in fp64 and
 * ranked, and the softmax uses those fp64 values, with the same certificate
 * and double-double fall-back. When `logits` is requested, all logits are
 * accumulated in fp64 (on the fp64 matrix cores beyond 64 tokens).
 *   X bf16 [T][H]; Wr fp32 [E][H]; bias fp32 [E] or NULL;
 *   idx int32 [T][k]; w fp32 [T][k]; logits fp32 [T][E] or NULL;
 *   n_fixup: int32 device scalar or NULL, receives the number of tokens that
 *   took the double-double path.
 * Limits: 1 <= k <= min(E, 16), E <= 1024, H in {256, 512, 1024, 2048, 4096}. */
size_t tmoe_router_workspace_bytes(int64_t T, int64_t E); /* fp64 logits, bound slots and (T >= 1024) the bf16
                                                              parts of the router rows for H up to 4096; no
                                                              zero-fill needed */
int tmoe_router_topk(void *stream, const uint16_t *X, int64_t T, int64_t H, const float *Wr, const float *bias,
                     int64_t E, int k, int32_t *idx, float *w, float *logits, int32_t *n_fixup, void *ws,
                     size_t ws_bytes);

/* ---------------------------------------------------------------- grouping
 * Stable token -> expert grouping of the T*k (token, slot) pairs: ordered by
 * expert, then token. counts [E]; offsets [E+1] (exclusive prefix sum,
 * offsets[E] = T*k); sorted_token, sorted_slot [T*k]; pos [T*k] with
 * pos[t*k + j] = grouped position of pair (t, j). Deterministic (no atomics
 * whose order matters). idx values must lie in [0, E) and a token must not
 * repeat an expert (the router guarantees both). */
size_t tmoe_group_workspace_bytes(int64_t T, int k, int64_t E);
int tmoe_group_by_expert(void *stream, const int32_t *idx, int64_t T, int k, int64_t E, int32_t *counts,
                         int32_t *offsets, int32_t *sorted_token, int32_t *sorted_slot, int32_t *pos, void *ws,
                         size_t ws_bytes);

/* ----------------------------------------------------------- layer weights */
typedef struct tmoe_moe_weights {
  int64_t hidden;    /* H, input/output width (2048) */
  int64_t inter;     /* I, moe_intermediate_size (512) */
  int64_t n_experts; /* E (256) */
  int32_t top_k;     /* k (8) */
  int32_t reserved;  /* must be 0 */
  const float *router_w;    /* fp32 [E][H] */
  const float *router_bias; /* fp32 [E] or NULL */
  /* Tiled packed expert weights; expert e's matrix starts at base + e * stride.
   * gate, up: [I][H] matrices; down: [H][I] matrices. */
  const uint8_t *gate_p;
  const uint8_t *up_p;
  const uint8_t *down_p;
  int64_t stride_gu; /* bytes between experts, >= tmoe_tiled_bytes(I, H) */
  int64_t stride_d;  /* bytes between experts, >= tmoe_tiled_bytes(H, I) */
  const float *gate_s; /* fp32 [E][I] */
  const float *up_s;   /* fp32 [E][I] */
  const float *down_s; /* fp32 [E][H] */
} tmoe_moe_weights;

/* ---------------------------------------------------------------- expert FFN
 * For every grouped pair p (expert e, token t = sorted_token[p]):
 *   g = gate_e x_t, u = up_e x_t            (ternary linear, fp32)
 *   h = SiLU(min(g, c)) * clamp(u, -c, c)   (c = clamp; INFINITY disables)
 *   O[p] = down_e h                          (ternary linear over fp32 h)
 * (ai.thesatyajit.com, "The shipped code does no quantization").
 * Precision: fp32 accumulation throughout. h enters the down projection
 * scaled per pair by a power of two 2^sig that puts the pair's largest |h| in
 * [2^14, 2^15), as two fp16 parts hi = fp16(2^sig h), lo = fp16(2^sig h - hi)
 * (22 of h's 24 significant bits; values under 2^-28 of the pair's largest
 * lose only bits below 2^-39 of it), multiplied exactly; the sums are
 * rescaled by 2^-sig exactly. This holds for every finite h, in both clamp
 * modes and at any input scale; results are finite whenever g, u, h and O
 * themselves are representable in fp32 (with the clamp on, |h| <= c SiLU(c)
 * for c >= 1.3, e.g. 49 for c = 7).
 *   X bf16 [T][H]; offsets [E+1], sorted_token [T*k] from the grouping;
 *   O fp32 [T*k][H] in grouped order; Hout fp32 [T*k][I] or NULL (h, for
 *   checking). ws: tmoe_ffn_workspace_bytes(T, W). */
size_t tmoe_ffn_workspace_bytes(int64_t T, const tmoe_moe_weights *W);
int tmoe_expert_ffn(void *stream, const tmoe_moe_weights *W, const uint16_t *X, int64_t T, const int32_t *offsets,
                    const int32_t *sorted_token, float clamp, float *O, float *Hout, void *ws, size_t ws_bytes);

/* ------------------------------------------------------------------ combine
 * Y[t] = sum_{j<k} w[t][j] * O[pos[t*k + j]] (fixed slot order, fp32), the
 * weighted sum of the k expert outputs (codeinsider.com.br, "256 experts, 8
 * ativos": 8 experts serve each token). If resid_out is not NULL, also
 * resid_out[t] = bf16_RNE(fp32(resid_in[t]) + Y[t]) (resid_in required then;
 * resid_out may alias resid_in). Y may be NULL when resid_out is given.
 *   O fp32 [T*k][H]; w fp32 [T][k]; pos int32 [T*k]; Y fp32 [T][H]. */
int tmoe_combine(void *stream, const float *O, const float *w, const int32_t *pos, int64_t T, int k, int64_t H,
                 float *Y, const uint16_t *resid_in, uint16_t *resid_out);

/* ------------------------------------------------------------- whole layer */
typedef struct tmoe_moe_options {
  float clamp;        /* activation clamp c; 7.0 in the model, INFINITY disables */
  int32_t reserved0;  /* must be 0 */
  /* Optional outputs (device, may be NULL): router results and grouping. */
  int32_t *idx;       /* [T][k] */
  float *w;           /* [T][k] */
  int32_t *pos;       /* [T*k]  */
  int32_t *n_fixup;   /* scalar */
  uint16_t *resid_out;/* [T][H] bf16: X + Y rounded to bf16 (the residual stream) */
} tmoe_moe_options;

/* Workspace bytes for tmoe_moe_forward with T tokens. Every call writes each
 * workspace byte it reads before reading it, so the workspace needs no
 * zero-fill and no per-call clearing (the call can be captured in a HIP
 * graph). Calls sharing one workspace must not run concurrently. */
int tmoe_moe_workspace_bytes(int64_t T, const tmoe_moe_weights *W, size_t *out);

/* The layer: router -> top-k -> grouping -> expert FFN -> combine.
 * X bf16 [T][H]; Y fp32 [T][H] (may be NULL if opt->resid_out is set).
 * opt may be NULL (clamp 7, no optional outputs).
 * Kernels: for T <= 3 (decode) three: fp64 router logits; gate/up whose
 * prologue certifies the top-k and groups the pairs; down with the combine
 * (and residual) fused. For T > 3: router logits, certified top-k, fix-up,
 * grouping, work tiles, gate/up, down, combine. */
int tmoe_moe_forward(void *stream, const tmoe_moe_weights *W, const uint16_t *X, int64_t T, float *Y,
                     const tmoe_moe_options *opt, void *ws, size_t ws_bytes);

/* Layer call for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and kernels as tmoe_moe_forward, with the workspace taken
 * from a fixed array of TMOE_NOALLOC_SCRATCH_BYTES in the library's own device
 * memory (one per GPU, reserved when the library's code is loaded on that
 * GPU and held until the process ends). Allocates nothing. The first call on a
 * device looks up that device's array (the calling thread's current device,
 * which must be the stream's). Requests whose workspace
 * (tmoe_moe_workspace_bytes) exceeds the array fail with TMOE_E_WORKSPACE
 * before anything is enqueued: at the model's shape (hidden 2048, 256 experts,
 * top 8, inter 512) up to 395 tokens fit. All calls on one GPU share its
 * array, so calls that may overlap on one GPU (different streams, or
 * different threads) race and must be serialized by the caller; each call
 * writes every byte of it that it reads, so nothing needs clearing between
 * calls. Arguments and errors otherwise as tmoe_moe_forward. */
#define TMOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int tmoe_moe_forward_noalloc(void *stream, const tmoe_moe_weights *W, const uint16_t *X, int64_t T, float *Y,
                             const tmoe_moe_options *opt);

/* ------------------------------------------------------- attention half
 * The step before the MoE in every layer (ai.thesatyajit.com, "The
 * architecture around the quantization"; jj-blog, architecture list): layers
 * repeat three sliding-window layers (a query sees the last 512 positions,
 * rotary embedding on half of each head: partial rotary factor 0.5) and one
 * global layer (the whole prefix, no positional encoding). The projections
 * are ternary like the experts; their sizes follow from the census (ai.
 * thesatyajit.com, "The 5.31 GB claim reconciles": 19.58B ternary weights
 * less the experts' 19.33B = 2 x 2048 x 2048 + 2 x 512 x 2048 per layer).
 * Head shape, rotary base and pairing are not on the pages and are fields here.
 * For tokens t = 0..T-1 at positions p = pos0 + t, with x = X[t]:
 *   [q; k; v] = s (.) (T_qkv x)            (query heads, then key, value heads)
 *   q, k rotated on sliding layers: pair (i, i + rotary_dim/2), i < rotary_dim/2,
 *        turns by p * rope_base^(-2i / rotary_dim)
 *   k, v of position p stored in cache slot p mod cache_cap
 *   attn_h = sum_j softmax_j(q_h . k_j / sqrt(head_dim)) v_j over the visible
 *        positions j of key/value head h / (n_heads / n_kv_heads): j <= p and,
 *        if window > 0, p - j < window
 *   O[t] = s_o (.) (T_o attn)               (attn fp32, split exactly into three bf16 parts)
 *   X_out[t] = bf16_RNE(fp32(x) + O[t])    (if X_out is not NULL)
 * Weights (device): qkv_p tiled [(n_heads + 2 n_kv_heads) head_dim][hidden],
 * qkv_s fp32 per row; o_p tiled [hidden][n_heads head_dim], o_s per row.
 * Cache (device, fp32, caller-owned): K and V [n_kv_heads][cache_cap][head_dim];
 * positions < pos0 must hold the keys and
 * values earlier calls stored. cache_cap >= pos0 + T (global layers) or
 * >= window + T - 1 (sliding: no slot a query of this call still sees is
 * overwritten). X bf16 [T][hidden], O fp32 [T][hidden] or NULL, X_out bf16
 * [T][hidden] or NULL (may alias X). Limits: hidden 2048, head_dim 128,
 * n_heads head_dim = hidden, n_heads = 4 n_kv_heads, rotary_dim even <= 128.
 * ws: tmoe_attention_workspace_bytes(T, W) bytes, no zero-fill; calls sharing
 * a workspace or a cache must not overlap. Errors: TMOE_E_ARG, TMOE_E_SHAPE
 * (cache too small, bad head shape), TMOE_E_ALIGN, TMOE_E_WORKSPACE,
 * TMOE_E_UNSUPPORTED. */
typedef struct tmoe_attn_weights {
  int64_t hidden;     /* 2048 */
  int32_t n_heads;    /* query heads (16) */
  int32_t n_kv_heads; /* key/value heads (4) */
  int32_t head_dim;   /* 128 */
  int32_t rotary_dim; /* rotated dimensions per head on sliding layers (64) */
  int32_t window;     /* > 0: sliding window (512), rotary; 0: global layer, no positional encoding */
  int32_t reserved;   /* must be 0 */
  double rope_base;   /* 10000 */
  const uint8_t *qkv_p;
  const float *qkv_s;
  const uint8_t *o_p;
  const float *o_s;
} tmoe_attn_weights;
size_t tmoe_attention_workspace_bytes(int64_t T, const tmoe_attn_weights *W);
int tmoe_attention_forward(void *stream, const tmoe_attn_weights *W, const uint16_t *X, int64_t T, int64_t pos0,
                           float *k_cache, float *v_cache, int64_t cache_cap, float *O, uint16_t *X_out, void *ws,
                           size_t ws_bytes);

/* --------------------------------------------------- host-resident experts
 * Page-locked host memory the GPU reads in place over PCIe. Expert weights
 * placed here (packed matrices and row scales; the router stays in HBM) are
 * fetched on demand by the layer's own kernels: a call moves only the bytes
 * of the experts its tokens select, and every step still runs on the GPU.
 * This is the MI355X form of keeping the experts off the device and streaming
 * the selected ones per layer (taozi.news, "Maple Preview 接入 Mference":
 * Mference, a turbo-fieldfare fork, leaves the experts on SSD and reads them
 * on demand). Fill the buffer, then pass `*device` addresses in
 * tmoe_moe_weights exactly as device memory; strides and layout are unchanged.
 *   bytes > 0; *host: CPU address of the buffer (write it before the first
 *   call that reads it, e.g. with hipMemcpy); *device: the address kernels use.
 * The memory is mapped and non-coherent (the GPU may cache what it reads), so
 * it must not change while any call that reads it may be in flight.
 * Errors: TMOE_E_ARG (zero size or null outputs), TMOE_E_HIP (allocation or
 * mapping failed; nothing is left allocated). tmoe_host_free releases a buffer
 * from tmoe_host_alloc (host address; NULL is a no-op); the device must not
 * be reading it. */
int tmoe_host_alloc(size_t bytes, void **host, void **device);
int tmoe_host_free(void *host);

/* ------------------------------------------------------------------ LM head
 * Output head over the vocabulary (ai.thesatyajit.com, "The 5.31 GB claim
 * reconciles, and the leftover is the vocabulary": the 151,936 x 2048 input
 * and output embeddings are untied and un-quantized; the output table alone
 * is 622 MB in bf16, the largest per-token byte stream of the model).
 *   logits[t][v] = sum_i X[t][i] * W[v][i]
 *   idx[t][0..k)  = the k largest logits, descending, equal logits -> lower v
 *   val[t][0..k)  = those logits (fp32 of the fp64 value)
 * Certified like the router: fp64 sums of exact products with a rigorous
 * error bound; equal fp64 logits of bitwise identical rows are exact ties;
 * any other top-(k+1) pair closer than the bound sends the token to a
 * double-double recompute of every token id within the bound of the
 * (k+1)-th logit. Indices equal those of the exact logits except for logits
 * closer than ~1e-30 relative.
 *   X bf16 [T][H]; W bf16 [V][H] (row-major, 16-B aligned); idx int32 [T][k];
 *   val fp32 [T][k]; logits fp32 [T][V] or NULL;
 *   n_fixup: int32 device scalar or NULL, incremented by the number of tokens
 *   ranked by the double-double path (and by 65536 for a token whose
 *   uncertain set exceeded 256 ids: that token keeps the float64 ranking).
 * Limits: T in {1, 2, 4} (decode), H in {512, 1024, 2048, 4096},
 * 1 <= k <= 16, k < V <= 2^20.
 * ws: tmoe_lm_head_workspace_bytes(T, V, k) bytes (fp64 logits, per-block
 * maxima, candidate lists); no zero-fill needed. Calls that share a
 * workspace must not overlap. */
size_t tmoe_lm_head_workspace_bytes(int64_t T, int64_t V, int k);
int tmoe_lm_head_topk(void *stream, const uint16_t *X, int64_t T, int64_t H, const uint16_t *W, int64_t V, int k,
                      int32_t *idx, float *val, float *logits, int32_t *n_fixup, void *ws, size_t ws_bytes);

/* ------------------------------------------------------------ kernel timing
 * Measurement hook. Between tmoe_profile_begin and tmoe_profile_end every
 * launch of one kernel (TMOE_KERNEL_*) carries a HIP start/stop event pair
 * that its own dispatch records on its stream (hipExtLaunchKernelGGL), for at
 * most `capacity` launches (later launches are not recorded). Before a timed
 * launch the host waits for its stream to drain, so the interval holds that
 * dispatch alone (the window is for measurement, never for throughput). Use it
 * on eager launches, not inside HIP graph capture. The events
 * are created by tmoe_profile_begin (not on the hot path) and destroyed by
 * tmoe_profile_end, which waits for them and writes the per-launch durations
 * in milliseconds to ms[0..*count). The events carry no system-scope fence
 * (hipEventDisableSystemFence), so they add no cache write-back to the timed
 * dispatch. The window belongs to the calling thread: only launches that
 * thread issues are timed, calls from other threads are untouched, and a
 * thread holds one window at a time (TMOE_E_ARG otherwise). */
enum {
  TMOE_KERNEL_ROUTER_LOGITS = 1, /* fp64 logits (VALU for T <= 64, matrix cores above) */
  TMOE_KERNEL_ROUTER_TOPK = 2,   /* certified top-k (with its rare double-double recompute) */
  TMOE_KERNEL_GROUP = 4,         /* the fused grouping kernel (first kernel when T > 256) */
  TMOE_KERNEL_MAKE_TILES = 5,    /* tmoe_expert_ffn only (the layer's grouping writes the tiles) */
  TMOE_KERNEL_GATEUP = 7,        /* for T <= 3 with the top-k and grouping in its prologue */
  TMOE_KERNEL_DOWN = 9,          /* for T*k <= 32 with the combine fused */
  TMOE_KERNEL_COMBINE = 10,
  TMOE_KERNEL_LINEAR = 11,
  TMOE_KERNEL_LMH_LOGITS = 12, /* LM head: the fp64 logit stream */
  TMOE_KERNEL_LMH_TOPK = 13,   /* LM head: per-chunk top-(k+1) */
  TMOE_KERNEL_LMH_MERGE = 14,  /* LM head: merge, certification, fallback */
  TMOE_KERNEL_ATTENTION = 15   /* attention half: the split softmax attention over the cache */
};
int tmoe_profile_begin(int kernel, int capacity);
int tmoe_profile_end(float *ms, int capacity, int *count);

#ifdef __cplusplus
}
#endif
#endif /* TMOE_H */
