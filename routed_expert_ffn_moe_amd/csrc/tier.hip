// Capacity-limited hot tier of expert records.
//
// The engine ships a usage profile that ranks every expert; each card fills its
// expert slots in that order, and an adaptive tier then swaps in at most 96
// experts every four rounds, towards the experts in actual use ("为什么 Strata
// 在小显存显卡上这么快", section "一台电脑就是一组水管"); the exponentially
// decayed usage score decides what is evicted ("Strata：12GB 显卡跑 125B 模型，
// MoE 专家热缓存打破 VRAM 限制", section "工作原理").
//
// Here the pool holds n_hot hot slots (0..n_hot-1) and every expert's record
// at its home slot (>= n_hot).  An expert is resident when a hot slot holds a
// copy of its record; the slot table then points at the copy, else at the
// home record, so the expert kernels read through the slot table unchanged.
// Both operations run on the device in one workgroup each, then a wide copy
// kernel moves the records.  The radix selects read their keys 9 times (8
// digit passes and a gather), so the keys are first cached in LDS when they
// fit (the 32-bit score keys of all L*E experts, and the hot slots' 64-bit
// victim keys); otherwise they are re-read from global memory.
//   fill:      the top n_hot experts by (score desc, flat index asc) become
//              resident, hot slot i holding the i-th of them in flat order
//              (radix select of the n_hot-th key, then a scan in flat order);
//   rebalance: the best-ranked experts that are not resident (candidates,
//              found by a radix select over the non-residents' rank keys)
//              replace the emptiest / lowest-scored hot slots (victims: empty
//              slots first, lower slot first, then score ascending, ties to
//              the higher flat index; a radix select over the hot slots)
//              while the slot is empty or the candidate scores strictly
//              higher, at most max_swaps of them.
#include "moe_common.h"
#include "moe_select.h"

#define TIER_CHUNK 65536  // bytes of a record copied by one workgroup
#define TIER_STATIC_LDS (20 * 1024)  // the kernels' static LDS, rounded up

extern __shared__ __attribute__((aligned(16))) uint8_t tier_lds[];

__device__ __forceinline__ int tier_row(int f, int E) { return (f / E) * (E + 1) + f % E; }

// rank order: score descending, flat index ascending (distinct keys)
__device__ __forceinline__ uint64_t tier_rank_key(const float* s, int f) {
  return ((uint64_t)moe_f32_order_key(s[f]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)f);
}

// Exclusive prefix sum of v over the 1024 threads (all threads call it).
__device__ int tier_block_exscan(int v, int* total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d, 64);
    if (lane >= d) incl += u;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0, all = 0;
  for (int w = 0; w < 16; ++w) {
    base += w < wave ? wsum[w] : 0;
    all += wsum[w];
  }
  __syncthreads();
  *total = all;
  return base + incl - v;
}

__global__ __launch_bounds__(1024) void tier_fill_kernel(const float* __restrict__ scores, int L, int E, int n_hot,
                                                         const int32_t* __restrict__ home, int32_t* slot,
                                                         int32_t* owner, int32_t* swaps, int32_t* n_swaps,
                                                         int cached) {
  const int N = L * E, tid = threadIdx.x;
  uint32_t* hi = (uint32_t*)tier_lds;  // [N] score keys when cached
  for (int i = tid; i < L * (E + 1); i += 1024) slot[i] = home[i];
  if (cached)
    for (int f = tid; f < N; f += 1024) hi[f] = moe_f32_order_key(scores[f]);
  __syncthreads();
  auto rank_key = [&](int f) -> uint64_t {
    return cached ? ((uint64_t)hi[f] << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)f) : tier_rank_key(scores, f);
  };
  const uint64_t thr = moe_kth_largest_key(rank_key, N, n_hot);
  // thread t scans flat indices [t C, (t+1) C): hot slots in flat order
  const int C = (N + 1023) / 1024;
  const int f0 = min(tid * C, N), f1 = min(f0 + C, N);
  int cnt = 0;
  for (int f = f0; f < f1; ++f) cnt += rank_key(f) >= thr;
  int total;
  int pos = tier_block_exscan(cnt, &total);  // its barriers also order the home copy above
  for (int f = f0; f < f1; ++f) {
    if (rank_key(f) >= thr) {
      const int r = tier_row(f, E);
      slot[r] = pos;
      owner[pos] = f;
      swaps[4 * pos + 0] = f;
      swaps[4 * pos + 1] = -1;
      swaps[4 * pos + 2] = pos;
      swaps[4 * pos + 3] = home[r];
      ++pos;
    }
  }
  if (tid == 0) *n_swaps = n_hot;
}

__global__ __launch_bounds__(1024) void tier_rebalance_kernel(const float* __restrict__ scores, int L, int E,
                                                              int n_hot, int max_swaps,
                                                              const int32_t* __restrict__ home, int32_t* slot,
                                                              int32_t* owner, int32_t* swaps, int32_t* n_swaps,
                                                              int cache_c, int cache_v) {
  __shared__ uint64_t csel[1024];
  __shared__ uint64_t sel[1024];
  __shared__ int nsw_s;
  const int tid = threadIdx.x, N = L * E;
  // residents: count the occupied hot slots
  int held = 0;
  for (int i = tid; i < n_hot; i += 1024) held += owner[i] >= 0;
  int n_held;
  tier_block_exscan(held, &n_held);
  const int m = min(min(N - n_held, max_swaps), n_hot);
  if (m == 0) {  // uniform over the workgroup
    if (tid == 0) *n_swaps = 0;
    return;
  }
  // LDS caches: chi[f] = the score key of expert f if it is not resident,
  // else 0; vk[i] = the victim key of hot slot i (below)
  uint32_t* chi = (uint32_t*)tier_lds;
  uint64_t* vk = (uint64_t*)(tier_lds + (cache_c ? ((size_t)N * 4 + 7) / 8 * 8 : 0));
  auto vkey = [&](int i) -> uint64_t {
    const int o = owner[i];
    if (o < 0) return (0xFFFFFFFFull << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)i);  // empty: lower slot first
    return ((uint64_t)(~moe_f32_order_key(scores[o])) << 32) | (uint32_t)o;            // low score, high index first
  };
  if (cache_c)
    for (int f = tid; f < N; f += 1024)
      chi[f] = slot[tier_row(f, E)] >= n_hot ? moe_f32_order_key(scores[f]) : 0u;
  if (cache_v)
    for (int i = tid; i < n_hot; i += 1024) vk[i] = vkey(i);
  __syncthreads();
  // candidates: the m best-ranked non-resident experts, in rank order (a
  // resident's key is 0, below every non-resident's, whose score keys are
  // nonzero; at least m are not resident)
  moe_top_keys_sorted(
      [&](int f) -> uint64_t {
        if (cache_c) return chi[f] ? ((uint64_t)chi[f] << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)f) : 0ull;
        return slot[tier_row(f, E)] >= n_hot ? tier_rank_key(scores, f) : 0ull;
      },
      N, m, csel);
  // victims: the m largest victim keys, in descending order
  moe_top_keys_sorted([&](int i) { return cache_v ? vk[i] : vkey(i); }, n_hot, m, sel);
  if (tid == 0) nsw_s = m;
  __syncthreads();
  int vslot = -1, vo = -1, cf = -1;
  if (tid < m) {
    const uint64_t k = sel[tid];
    const uint32_t hi = (uint32_t)(k >> 32), lo = (uint32_t)k;
    if (hi == 0xFFFFFFFFu) {
      vslot = (int)(0xFFFFFFFFu - lo);
    } else {
      vo = (int)lo;
      vslot = slot[tier_row(vo, E)];
    }
    cf = (int)(0xFFFFFFFFu - (uint32_t)csel[tid]);
    // candidates descend and victims ascend in score: the first pair that
    // does not improve ends the swaps
    if (!(vo < 0 || scores[cf] > scores[vo])) atomicMin(&nsw_s, tid);
  }
  __syncthreads();  // every read of slot[] above happens before the writes below
  const int nsw = nsw_s;
  if (tid < nsw) {
    const int rc = tier_row(cf, E);
    slot[rc] = vslot;
    if (vo >= 0) slot[tier_row(vo, E)] = home[tier_row(vo, E)];
    owner[vslot] = cf;
    swaps[4 * tid + 0] = cf;
    swaps[4 * tid + 1] = vo;
    swaps[4 * tid + 2] = vslot;
    swaps[4 * tid + 3] = home[rc];
  }
  if (tid == 0) *n_swaps = nsw;
}

// Record copies: workgroup b copies chunk b % nchunks of swap b / nchunks
// (swaps past *n_swaps do nothing), 4 16-byte words per thread in flight.
__global__ __launch_bounds__(256) void tier_copy_kernel(uint8_t* pool, int64_t R, const int32_t* __restrict__ swaps,
                                                        const int32_t* __restrict__ n_swaps, int nchunks) {
  const int s = blockIdx.x / nchunks, ch = blockIdx.x % nchunks;
  if (s >= *n_swaps) return;
  const int64_t src = swaps[4 * s + 3], dst = swaps[4 * s + 2];
  const int64_t w0 = (int64_t)ch * (TIER_CHUNK / 16);
  const int64_t w1 = w0 + TIER_CHUNK / 16 < R / 16 ? w0 + TIER_CHUNK / 16 : R / 16;
  const uint4* in = reinterpret_cast<const uint4*>(pool + src * R);
  uint4* out = reinterpret_cast<uint4*>(pool + dst * R);
  for (int64_t i = w0 + threadIdx.x; i < w1; i += 4 * 256) {
    // four named registers (an array here was placed in LDS by the compiler)
    const uint4 zero = {0u, 0u, 0u, 0u};
    const uint4 v0 = in[i];
    const uint4 v1 = i + 256 < w1 ? in[i + 256] : zero;
    const uint4 v2 = i + 512 < w1 ? in[i + 512] : zero;
    const uint4 v3 = i + 768 < w1 ? in[i + 768] : zero;
    out[i] = v0;
    if (i + 256 < w1) out[i + 256] = v1;
    if (i + 512 < w1) out[i + 512] = v2;
    if (i + 768 < w1) out[i + 768] = v3;
  }
}

static size_t tier_lds_limit() {
  static size_t lim = 0;
  if (!lim) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeSharedMemPerBlockOptin, dev) == hipSuccess && v > 0)
      lim = (size_t)v;
    else
      lim = 64 * 1024;
  }
  return lim;
}

static int tier_set_lds(const void* fn, size_t bytes) {
  if (bytes == 0) return MOE_OK;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) != hipSuccess)
    return moe_fail(MOE_EHIP, "tier: cannot reserve %zu bytes of LDS", bytes);
  return MOE_OK;
}

static int tier_launch_copy(void* pool, int64_t R, int32_t* swaps, int32_t* n_swaps, int max_swaps, hipStream_t st) {
  if (max_swaps <= 0) return MOE_OK;
  const int nchunks = (int)((R + TIER_CHUNK - 1) / TIER_CHUNK);
  tier_copy_kernel<<<(unsigned)max_swaps * (unsigned)nchunks, 256, 0, st>>>((uint8_t*)pool, R, swaps, n_swaps,
                                                                             nchunks);
  return MOE_OK;
}

#define TIER_COMMON_CHECKS()                                                                                     \
  MOE_REQUIRE(L >= 1 && E >= 1 && E <= MOE_MAX_E && (int64_t)L * E <= 65536, MOE_ESHAPE,                          \
              "L*E must be in [1, 65536] with E <= %d", MOE_MAX_E);                                                \
  MOE_REQUIRE(n_hot >= 1 && n_hot <= L * E, MOE_ESHAPE, "n_hot=%d out of [1, L*E]", n_hot);                         \
  MOE_REQUIRE(record_bytes > 0 && record_bytes % 256 == 0, MOE_EALIGN, "record_bytes must be a positive multiple of 256"); \
  MOE_REQUIRE(((uintptr_t)pool & 255) == 0, MOE_EALIGN, "pool must be 256-byte aligned");                           \
  MOE_REQUIRE(scores && home_table && slot_table && hot_owner && pool && swaps && n_swaps, MOE_EINVAL,           \
              "every pointer is required")

extern "C" int moe_tier_fill(const float* scores, int L, int E, int n_hot, const int32_t* home_table,
                             int32_t* slot_table, int32_t* hot_owner, void* pool, int64_t record_bytes,
                             int32_t* swaps, int32_t* n_swaps, void* stream) {
  TIER_COMMON_CHECKS();
  hipStream_t st = moe_stream(stream);
  const size_t need = (size_t)L * E * 4;
  const int cached = need + TIER_STATIC_LDS <= tier_lds_limit();
  const size_t lds = cached ? need : 0;
  if (tier_set_lds((const void*)tier_fill_kernel, lds) != MOE_OK) return MOE_EHIP;
  tier_fill_kernel<<<1, 1024, lds, st>>>(scores, L, E, n_hot, home_table, slot_table, hot_owner, swaps, n_swaps,
                                         cached);
  tier_launch_copy(pool, record_bytes, swaps, n_swaps, n_hot, st);
  return moe_check_launch("tier fill");
}

extern "C" int moe_tier_rebalance(const float* scores, int L, int E, int n_hot, int max_swaps,
                                  const int32_t* home_table, int32_t* slot_table, int32_t* hot_owner, void* pool,
                                  int64_t record_bytes, int32_t* swaps, int32_t* n_swaps, void* stream) {
  TIER_COMMON_CHECKS();
  MOE_REQUIRE(max_swaps >= 0 && max_swaps <= 1024, MOE_ESHAPE, "max_swaps=%d out of [0, 1024]", max_swaps);
  hipStream_t st = moe_stream(stream);
  const size_t need_c = ((size_t)L * E * 4 + 7) / 8 * 8, need_v = (size_t)n_hot * 8, lim = tier_lds_limit();
  const int cache_c = need_c + TIER_STATIC_LDS <= lim;
  const int cache_v = (cache_c ? need_c : 0) + need_v + TIER_STATIC_LDS <= lim;
  const size_t lds = (cache_c ? need_c : 0) + (cache_v ? need_v : 0);
  if (tier_set_lds((const void*)tier_rebalance_kernel, lds) != MOE_OK) return MOE_EHIP;
  tier_rebalance_kernel<<<1, 1024, lds, st>>>(scores, L, E, n_hot, max_swaps, home_table, slot_table, hot_owner,
                                              swaps, n_swaps, cache_c, cache_v);
  tier_launch_copy(pool, record_bytes, swaps, n_swaps, min(max_swaps, n_hot), st);
  return moe_check_launch("tier rebalance");
}
