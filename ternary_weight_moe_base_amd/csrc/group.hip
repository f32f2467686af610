// Deterministic token -> expert grouping.
//
// Each token is served by k of E experts (codeinsider.com.br, "256 experts, 8
// ativos"); the expert kernels need the (token, slot) pairs grouped by expert.
// Pairs are ordered by expert, then token. A pair's position is
//   offsets[e] + (pairs of e in earlier token blocks) + (tokens before t in
//   its block that chose e),
// the last term read from a per-block bitmask of the tokens choosing each
// expert (popcount of the bits below t). No atomics influence any output
// value or order (the bitmask is built with atomicOr, which commutes).
#include "device_util.h"

namespace tmoe {

static constexpr int kBlockTok = 256;  // tokens per grouping block = threads per workgroup

size_t group_ws_bytes(int64_t T, int k, int64_t E) {
  (void)k;
  int64_t nb = cdiv(T, kBlockTok);
  if (nb <= 1) return 0;
  return 2 * align_up((size_t)nb * E * 4, 256);
}

GroupWs group_ws_carve(void *ws, int64_t T, int k, int64_t E) {
  (void)k;
  GroupWs g{nullptr, nullptr};
  int64_t nb = cdiv(T, kBlockTok);
  if (nb <= 1 || !ws) return g;
  g.bcount = (int32_t *)ws;
  g.bbase = (int32_t *)((char *)ws + align_up((size_t)nb * E * 4, 256));
  return g;
}

// bits[e * 8 + w]: bit b set <=> token (block_start + 32 w + b) chose expert e.
__device__ inline void build_bitmask(uint32_t *bits, const int32_t *idx, int64_t T, int k, int E, int64_t t0) {
  for (int i = threadIdx.x; i < E * 8; i += kBlockTok) bits[i] = 0;
  __syncthreads();
  const int64_t t = t0 + threadIdx.x;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      int e = idx[t * k + j];
      if (e >= 0 && e < E) atomicOr(&bits[e * 8 + (threadIdx.x >> 5)], 1u << (threadIdx.x & 31));
    }
  }
  __syncthreads();
}

__device__ inline int block_count(const uint32_t *bits, int e) {
  int c = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) c += __popc(bits[e * 8 + w]);
  return c;
}

// rank of token slot `tid` among the block's tokens that chose e
__device__ inline int block_rank(const uint32_t *bits, int e, int tid) {
  int w = tid >> 5, r = 0;
  for (int i = 0; i < w; ++i) r += __popc(bits[e * 8 + i]);
  return r + __popc(bits[e * 8 + w] & ((1u << (tid & 31)) - 1u));
}

__device__ inline void scatter_block(const uint32_t *bits, const int *base, const int32_t *idx, int64_t T, int k,
                                     int E, int64_t t0, int32_t *sorted_token, int32_t *sorted_slot, int32_t *pos) {
  const int64_t t = t0 + threadIdx.x;
  if (t >= T) return;
  for (int j = 0; j < k; ++j) {
    int e = idx[t * k + j];
    int p = -1;
    if (e >= 0 && e < E) {
      p = base[e] + block_rank(bits, e, threadIdx.x);
      sorted_token[p] = (int32_t)t;
      sorted_slot[p] = j;
    }
    pos[t * k + j] = p;
  }
}

// k <= KM (the layer's top-k): a thread reads its token's k choices once, all
// loads in flight together, and builds the bitmask and scatters from
// registers (the generic loops above reload idx after every store, since the
// stores may alias it).
template <int KM>
__device__ inline void load_choices(const int32_t *idx, int64_t T, int k, int64_t t0, int (&ch)[KM]) {
  const int64_t t = t0 + threadIdx.x;
#pragma unroll
  for (int j = 0; j < KM; ++j) ch[j] = (t < T && j < k) ? idx[t * k + j] : -1;
}

template <int KM>
__device__ inline void build_bitmask_r(uint32_t *bits, const int (&ch)[KM], int E) {
  for (int i = threadIdx.x; i < E * 8; i += kBlockTok) bits[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const int e = ch[j];
    if (e >= 0 && e < E) atomicOr(&bits[e * 8 + (threadIdx.x >> 5)], 1u << (threadIdx.x & 31));
  }
  __syncthreads();
}

template <int KM>
__device__ inline void scatter_block_r(const uint32_t *bits, const int *base, const int (&ch)[KM], int64_t T, int k,
                                       int E, int64_t t0, int32_t *sorted_token, int32_t *sorted_slot, int32_t *pos) {
  const int64_t t = t0 + threadIdx.x;
  if (t >= T) return;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j >= k) break;
    const int e = ch[j];
    int p = -1;
    if (e >= 0 && e < E) {
      p = base[e] + block_rank(bits, e, threadIdx.x);
      sorted_token[p] = (int32_t)t;
      sorted_slot[p] = j;
    }
    pos[t * k + j] = p;
  }
}

// Work tiles of up to `tile` grouped pairs of one expert, in expert order,
// from the per-expert counts c[] and offsets off[] (tc[], tmp[]: LDS scratch).
__device__ inline void write_tiles(const int *c, const int *off, int E, int *tc, int *tmp, int32_t *tiles,
                                   int32_t *ntiles, int tile) {
  for (int e = threadIdx.x; e < E; e += kBlockTok) tc[e] = (c[e] + tile - 1) / tile;
  __syncthreads();
  const int total = block_exclusive_scan<kBlockTok>(tc, E, tmp);
  for (int e = threadIdx.x; e < E; e += kBlockTok)
    for (int i = 0; tile * i < c[e]; ++i)
      reinterpret_cast<int4 *>(tiles)[tc[e] + i] = make_int4(e, off[e] + tile * i, min(tile, c[e] - tile * i), 0);
  if (threadIdx.x == 0) *ntiles = total;
}

// Whole grouping in one workgroup (T <= 256). KM > 0: k <= KM, choices in registers.
template <int KM>
__global__ __launch_bounds__(kBlockTok) void group_fused_kernel(const int32_t *idx, int64_t T, int k, int E,
                                                                int32_t *counts, int32_t *offsets,
                                                                int32_t *sorted_token, int32_t *sorted_slot,
                                                                int32_t *pos, int32_t *tiles, int32_t *ntiles,
                                                                int tile) {
  __shared__ uint32_t bits[1024 * 8];
  __shared__ int cnt[1024], c0[1024], tc[1024];
  __shared__ int tmp[kBlockTok];
  int ch[KM > 0 ? KM : 1];
  if constexpr (KM > 0) {
    load_choices<KM>(idx, T, k, 0, ch);
    build_bitmask_r<KM>(bits, ch, E);
  } else {
    build_bitmask(bits, idx, T, k, E, 0);
  }
  for (int e = threadIdx.x; e < E; e += kBlockTok) {
    int c = block_count(bits, e);
    cnt[e] = c;
    c0[e] = c;
    counts[e] = c;
  }
  __syncthreads();
  int total = block_exclusive_scan<kBlockTok>(cnt, E, tmp);
  for (int e = threadIdx.x; e < E; e += kBlockTok) offsets[e] = cnt[e];
  if (threadIdx.x == 0) offsets[E] = total;
  if constexpr (KM > 0)
    scatter_block_r<KM>(bits, cnt, ch, T, k, E, 0, sorted_token, sorted_slot, pos);
  else
    scatter_block(bits, cnt, idx, T, k, E, 0, sorted_token, sorted_slot, pos);
  if (tiles) write_tiles(c0, cnt, E, tc, tmp, tiles, ntiles, tile);
}

template <int KM>
__global__ __launch_bounds__(kBlockTok) void group_count_kernel(const int32_t *idx, int64_t T, int k, int E,
                                                                int32_t *bcount) {
  __shared__ uint32_t bits[1024 * 8];
  if constexpr (KM > 0) {
    int ch[KM];
    load_choices<KM>(idx, T, k, (int64_t)blockIdx.x * kBlockTok, ch);
    build_bitmask_r<KM>(bits, ch, E);
  } else {
    build_bitmask(bits, idx, T, k, E, (int64_t)blockIdx.x * kBlockTok);
  }
  for (int e = threadIdx.x; e < E; e += kBlockTok) bcount[(int64_t)blockIdx.x * E + e] = block_count(bits, e);
}

// Per expert, the block counts are read 16 blocks at a time, all 16 loads in
// flight before the running sum is stored (stores to bbase may alias bcount as
// far as the compiler knows, so a load after each store would wait for it).
__global__ __launch_bounds__(kBlockTok) void group_scan_kernel(const int32_t *bcount, int nb, int E, int32_t *bbase,
                                                               int32_t *counts, int32_t *offsets, int32_t *tiles,
                                                               int32_t *ntiles, int tile) {
  constexpr int B = 16;
  __shared__ int cnt[1024], c0[1024], tc[1024];
  __shared__ int tmp[kBlockTok];
  for (int e = threadIdx.x; e < E; e += kBlockTok) {
    int run = 0;
    for (int b0 = 0; b0 < nb; b0 += B) {
      int c[B];
#pragma unroll
      for (int u = 0; u < B; ++u) c[u] = bcount[(int64_t)min(b0 + u, nb - 1) * E + e];
#pragma unroll
      for (int u = 0; u < B; ++u)
        if (b0 + u < nb) {
          bbase[(int64_t)(b0 + u) * E + e] = run;
          run += c[u];
        }
    }
    cnt[e] = run;
    c0[e] = run;
    counts[e] = run;
  }
  __syncthreads();
  int total = block_exclusive_scan<kBlockTok>(cnt, E, tmp);
  for (int e = threadIdx.x; e < E; e += kBlockTok) offsets[e] = cnt[e];
  if (threadIdx.x == 0) offsets[E] = total;
  if (tiles) write_tiles(c0, cnt, E, tc, tmp, tiles, ntiles, tile);
}

template <int KM>
__global__ __launch_bounds__(kBlockTok) void group_scatter_kernel(const int32_t *idx, int64_t T, int k, int E,
                                                                  const int32_t *offsets, const int32_t *bbase,
                                                                  int32_t *sorted_token, int32_t *sorted_slot,
                                                                  int32_t *pos) {
  __shared__ uint32_t bits[1024 * 8];
  __shared__ int base[1024];
  for (int e = threadIdx.x; e < E; e += kBlockTok) base[e] = offsets[e] + bbase[(int64_t)blockIdx.x * E + e];
  const int64_t t0 = (int64_t)blockIdx.x * kBlockTok;
  if constexpr (KM > 0) {
    int ch[KM];
    load_choices<KM>(idx, T, k, t0, ch);
    build_bitmask_r<KM>(bits, ch, E);
    scatter_block_r<KM>(bits, base, ch, T, k, E, t0, sorted_token, sorted_slot, pos);
  } else {
    build_bitmask(bits, idx, T, k, E, t0);
    scatter_block(bits, base, idx, T, k, E, t0, sorted_token, sorted_slot, pos);
  }
}

// Scatter with the scan folded in, for a batch of a few token blocks (at most
// kScanInMaxBlocks): each workgroup reads the block counts of every expert
// (group_count_kernel's output), forms the expert totals, the pairs in blocks
// before its own and the expert offsets (one workgroup scan), then scatters
// its block as group_scatter_kernel does from the same bases. Workgroup 0 also
// writes counts, offsets and the work tiles. Same outputs as scan + scatter,
// one launch fewer.
static constexpr int kScanInMaxBlocks = 64;

template <int KM>
__global__ __launch_bounds__(kBlockTok) void group_scatter_scan_kernel(const int32_t *idx, int64_t T, int k, int E,
                                                                       const int32_t *bcount, int nb, int32_t *counts,
                                                                       int32_t *offsets, int32_t *sorted_token,
                                                                       int32_t *sorted_slot, int32_t *pos,
                                                                       int32_t *tiles, int32_t *ntiles, int tile) {
  constexpr int B = 16;
  __shared__ uint32_t bits[1024 * 8];
  __shared__ int off[1024], base[1024], c0[1024], tc[1024];
  __shared__ int tmp[kBlockTok];
  const int64_t t0 = (int64_t)blockIdx.x * kBlockTok;
  // this workgroup's own choices first, in flight with the counts
  int ch[KM > 0 ? KM : 1];
  if constexpr (KM > 0) load_choices<KM>(idx, T, k, t0, ch);
  for (int e = threadIdx.x; e < E; e += kBlockTok) {
    int tot = 0, before = 0;
    for (int b0 = 0; b0 < nb; b0 += B) {
      int c[B];
#pragma unroll
      for (int u = 0; u < B; ++u) c[u] = bcount[(int64_t)min(b0 + u, nb - 1) * E + e];
#pragma unroll
      for (int u = 0; u < B; ++u) {
        tot += b0 + u < nb ? c[u] : 0;
        before += b0 + u < (int)blockIdx.x ? c[u] : 0;
      }
    }
    off[e] = tot;
    c0[e] = tot;
    base[e] = before;
    if (blockIdx.x == 0) counts[e] = tot;
  }
  const int total = block_exclusive_scan<kBlockTok>(off, E, tmp);  // off: expert offsets
  for (int e = threadIdx.x; e < E; e += kBlockTok) {
    base[e] += off[e];
    if (blockIdx.x == 0) offsets[e] = off[e];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) offsets[E] = total;
  if constexpr (KM > 0) {
    build_bitmask_r<KM>(bits, ch, E);  // its first barrier also orders the base writes above
    scatter_block_r<KM>(bits, base, ch, T, k, E, t0, sorted_token, sorted_slot, pos);
  } else {
    build_bitmask(bits, idx, T, k, E, t0);
    scatter_block(bits, base, idx, T, k, E, t0, sorted_token, sorted_slot, pos);
  }
  if (blockIdx.x == 0 && tiles) write_tiles(c0, off, E, tc, tmp, tiles, ntiles, tile);
}

template <int KM>
static int launch_group_k(hipStream_t st, const int32_t *idx, int64_t T, int k, int64_t E, int32_t *counts,
                          int32_t *offsets, int32_t *sorted_token, int32_t *sorted_slot, int32_t *pos,
                          const GroupWs &gw, int32_t *tiles, int32_t *ntiles, int tile) {
  const int64_t nb = cdiv(T, kBlockTok);
  if (nb <= 1) {
    TMOE_LAUNCH(TMOE_KERNEL_GROUP, group_fused_kernel<KM>, dim3(1), dim3(kBlockTok), 0, st, idx, T, k, (int)E, counts,
                offsets, sorted_token, sorted_slot, pos, tiles, ntiles, tile);
    TMOE_LAUNCHED("group_fused");
    return TMOE_OK;
  }
  if (nb > 0x7FFFFFFF) return fail(TMOE_E_UNSUPPORTED, "T too large");
  TMOE_LAUNCH(TMOE_KERNEL_GROUP, group_count_kernel<KM>, dim3((unsigned)nb), dim3(kBlockTok), 0, st, idx, T, k, (int)E,
              gw.bcount);
  TMOE_LAUNCHED("group_count");
  if (nb <= kScanInMaxBlocks) {
    hipLaunchKernelGGL(group_scatter_scan_kernel<KM>, dim3((unsigned)nb), dim3(kBlockTok), 0, st, idx, T, k, (int)E,
                       gw.bcount, (int)nb, counts, offsets, sorted_token, sorted_slot, pos, tiles, ntiles, tile);
    TMOE_LAUNCHED("group_scatter_scan");
    return TMOE_OK;
  }
  hipLaunchKernelGGL(group_scan_kernel, dim3(1), dim3(kBlockTok), 0, st, gw.bcount, (int)nb, (int)E, gw.bbase, counts,
                     offsets, tiles, ntiles, tile);
  TMOE_LAUNCHED("group_scan");
  hipLaunchKernelGGL(group_scatter_kernel<KM>, dim3((unsigned)nb), dim3(kBlockTok), 0, st, idx, T, k, (int)E, offsets,
                     gw.bbase, sorted_token, sorted_slot, pos);
  TMOE_LAUNCHED("group_scatter");
  return TMOE_OK;
}

int launch_group(hipStream_t st, const int32_t *idx, int64_t T, int k, int64_t E, int32_t *counts, int32_t *offsets,
                 int32_t *sorted_token, int32_t *sorted_slot, int32_t *pos, const GroupWs &gw, int32_t *tiles,
                 int32_t *ntiles, int tile) {
  if (tiles && tile < 1) return fail(TMOE_E_ARG, "tile size %d", tile);
  if (k <= 8)
    return launch_group_k<8>(st, idx, T, k, E, counts, offsets, sorted_token, sorted_slot, pos, gw, tiles, ntiles,
                             tile);
  if (k <= 16)
    return launch_group_k<16>(st, idx, T, k, E, counts, offsets, sorted_token, sorted_slot, pos, gw, tiles, ntiles,
                              tile);
  return launch_group_k<0>(st, idx, T, k, E, counts, offsets, sorted_token, sorted_slot, pos, gw, tiles, ntiles, tile);
}

}  // namespace tmoe
