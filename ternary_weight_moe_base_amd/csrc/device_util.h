// Device helpers shared by the .hip sources of libtmoe.
#pragma once

#include "common.h"

namespace tmoe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// s_waitcnt with only the vector-memory count (expcnt and lgkmcnt not waited)
#define TMOE_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
// Buffer resource word 3 for raw (untyped) buffer accesses on gfx9-family parts
constexpr int kBufWord3 = 0x00020000;

// 16 bytes from LDS (one matrix-core operand of a lane)
__device__ __forceinline__ u32x4 lds16(const char *p) { return *reinterpret_cast<const u32x4 *>(p); }

struct KeepChunk {
  __device__ uint4 operator()(int, uint4 v) const { return v; }
};

// Copies n 16-byte chunks, chunk i from *src(i) to *dst(i) (through
// fix(i, value)), by a workgroup of NT threads with up to 8 loads in flight per
// thread: all loads of a batch are issued before its stores.
template <int NT, typename Src, typename Dst, typename Fix = KeepChunk>
__device__ inline void copy16(int n, Src src, Dst dst, Fix fix = Fix()) {
  constexpr int B = 8;
  for (int base = threadIdx.x; base < n; base += NT * B) {
    uint4 v[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int i = base + j * NT;
      if (i < n) v[j] = src(i);
    }
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int i = base + j * NT;
      if (i < n) *dst(i) = fix(i, v[j]);
    }
  }
}

// Exclusive prefix sum of cnt[0..n) in place by a workgroup of NT threads
// (NT a multiple of 64, n <= 4 * NT); tmp holds NT ints. Returns the total to
// every thread. Each thread sums a run of consecutive entries, the runs are
// scanned within each wavefront by shuffles and across wavefronts through
// tmp: three barriers.
template <int NT>
__device__ inline int block_exclusive_scan(int *cnt, int n, int *tmp) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per = (n + NT - 1) / NT;
  const int b0 = threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (b0 + i < n) local += cnt[b0 + i];
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int tw = tmp[w];
    before += w < wave ? tw : 0;
    total += tw;
  }
  int run = before + incl - local;
  for (int i = 0; i < per; ++i)
    if (b0 + i < n) {
      const int c = cnt[b0 + i];
      cnt[b0 + i] = run;
      run += c;
    }
  __syncthreads();
  return total;
}

// Round a finite fp32 value to bf16, nearest even; returns the bit pattern.
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// LDS accesses of this wavefront done, then the workgroup barrier. Unlike
// __syncthreads() it does not wait for the wavefront's global loads and stores
// in flight (vmcnt), so they may cross the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

}  // namespace tmoe
