// Selection among distinct 64-bit keys by one workgroup of 1024 threads.
#pragma once
#include "moe_common.h"

// The n-th largest of the N distinct keys key(0..N-1), 1 <= n <= N: an
// 8-pass MSB radix select (a 256-bin LDS histogram of the next byte among the
// keys that share the bytes fixed so far).  Exactly n keys are >= the result.
// Called by all 1024 threads of the workgroup; returns the same value in each.
// Keys often share their leading bytes (scores of similar size), so in each
// wave the lanes holding the first active lane's digit add their count with
// one atomic; the other lanes add one each.
template <class KeyF>
__device__ uint64_t moe_kth_largest_key(KeyF key, int N, int n) {
  __shared__ __attribute__((aligned(16))) unsigned hist[256];
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
    for (int i0 = 0; i0 < N; i0 += 1024) {  // uniform trip count: whole waves take part
      const int i = i0 + tid;
      const uint64_t k = i < N ? key(i) : 0ull;
      const bool act = i < N && (k & hi_mask) == prefix;
      const unsigned d = (unsigned)(k >> shift) & 255u;
      const uint64_t live = __ballot(act);
      if (live) {  // wave-uniform
        const int lead = __ffsll((long long)live) - 1;
        const unsigned dl = (unsigned)__shfl((int)d, lead, 64);
        const uint64_t same = __ballot(act && d == dl);
        if ((tid & 63) == lead) atomicAdd(&hist[dl], (unsigned)__popcll(same));
        if (act && d != dl) atomicAdd(&hist[d], 1u);
      }
    }
    __syncthreads();
    if (tid < 64) {
      // the largest digit d whose suffix count (keys with digit >= d) reaches
      // `need`, by one wave: lane l holds bins 4l..4l+3
      const uint4 hb = *reinterpret_cast<const uint4*>(&hist[4 * tid]);
      const int own = (int)(hb.x + hb.y + hb.z + hb.w);
      int suf = own;  // sum over lanes >= tid
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_down(suf, off, 64);
        suf += tid + off < 64 ? v : 0;
      }
      const int s3 = suf - own + (int)hb.w, s2 = s3 + (int)hb.z, s1 = s2 + (int)hb.y, s0 = s1 + (int)hb.x;
      const int best = s3 >= need ? 3 : s2 >= need ? 2 : s1 >= need ? 1 : s0 >= need ? 0 : -1;
      const uint64_t has = __ballot(best >= 0);
      const int win = has ? 63 - __clzll((long long)has) : 0;  // the highest lane (digit 0 if none)
      if (tid == win) {
        const int dd = best >= 0 ? best : 0;
        const int sd = dd == 3 ? s3 : dd == 2 ? s2 : dd == 1 ? s1 : s0;
        const unsigned hd = dd == 3 ? hb.w : dd == 2 ? hb.z : dd == 1 ? hb.y : hb.x;
        prefix_s = prefix | ((uint64_t)(4 * tid + dd) << shift);
        need_s = need - (sd - (int)hd);  // minus the keys above digit d
      }
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
// it gathered, then a bitonic sort over the P entries, P the power of two
// >= n (entries n..P-1 zero).
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
  int P = 2;
  while (P < n) P <<= 1;
  if (tid >= cnt_s && tid < P) sel[tid] = 0ull;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int j = tid ^ stride;
      if (tid < P && j > tid) {
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
