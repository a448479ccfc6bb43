// Selection among distinct 64-bit keys by one workgroup of 1024 threads.
#pragma once
#include "moe_common.h"

// The n-th largest of the N distinct keys key(0..N-1), 1 <= n <= N: an
// 8-pass MSB radix select (a 256-bin LDS histogram of the next byte among the
// keys that share the bytes fixed so far).  Exactly n keys are >= the result.
// Called by all 1024 threads of the workgroup; returns the same value in each.
template <class KeyF>
__device__ uint64_t moe_kth_largest_key(KeyF key, int N, int n) {
  __shared__ unsigned hist[256];
  __shared__ uint64_t prefix_s;
  __shared__ int need_s;
  const int tid = threadIdx.x;
  uint64_t prefix = 0;
  int need = n;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    const uint64_t hi_mask = pass == 0 ? 0ull : (~0ull << (shift + 8));
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < N; i += 1024) {
      const uint64_t k = key(i);
      if ((k & hi_mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int above = 0, d = 255;
      for (; d > 0; --d) {
        if (above + (int)hist[d] >= need) break;
        above += hist[d];
      }
      prefix_s = prefix | ((uint64_t)d << shift);
      need_s = need - above;
    }
    __syncthreads();
    prefix = prefix_s;
    need = need_s;
    __syncthreads();
  }
  return prefix;
}

// The n largest keys in descending order into sel[0..n-1] (LDS, 1024
// entries; 1 <= n <= min(N, 1024)): the threshold above, the keys at or above
// it gathered, then a bitonic sort over the 1024 entries (the rest zero).
template <class KeyF>
__device__ void moe_top_keys_sorted(KeyF key, int N, int n, uint64_t* sel) {
  __shared__ int cnt_s;
  const int tid = threadIdx.x;
  const uint64_t thr = moe_kth_largest_key(key, N, n);
  if (tid == 0) cnt_s = 0;
  __syncthreads();
  for (int i = tid; i < N; i += 1024) {
    const uint64_t k = key(i);
    if (k >= thr) sel[atomicAdd(&cnt_s, 1)] = k;
  }
  __syncthreads();
  if (tid >= cnt_s) sel[tid] = 0ull;
  __syncthreads();
  for (int size = 2; size <= 1024; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int j = tid ^ stride;
      if (j > tid) {
        const bool desc = (tid & size) == 0;
        const uint64_t a = sel[tid], b = sel[j];
        if (desc ? (a < b) : (a > b)) {
          sel[tid] = b;
          sel[j] = a;
        }
      }
      __syncthreads();
    }
  }
}
