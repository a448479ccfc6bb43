// Stable permutation of the (token, choice) pairs by expert: histogram,
// exclusive scan, scatter.  A prefill chunk routes to nearly every expert of
// the layer ("为什么 Strata 在小显存显卡上这么快", section "读长提示词：大块流式
// 读取"); grouping the pairs by expert lets one read of an expert's weights
// serve all its tokens.
//
// The pairs are cut into chunks of MOE_PERMUTE_CHUNK in flat order t*k+j.
//   1. per chunk: count the experts (LDS integer atomics; order-free).
//   2. one workgroup: per expert, exclusive prefix over chunks, then an
//      exclusive scan over experts -> offsets and each chunk's base row.
//   3. per chunk, eight waves each walk an eighth of it in order, 64 pairs at
//      a time, from per-expert rows offset by the eighths before; lanes holding
//      the same expert find each other with bit-sliced ballots, so the rank
//      inside a batch is the number of lower lanes with that expert.
// Every step is integer and order-deterministic, so the result is bit-exact.
#include "moe_common.h"
#include "moe_sizes.h"

__global__ __launch_bounds__(256) void permute_hist_kernel(const int32_t* __restrict__ idx, int n, int E,
                                                           int32_t* __restrict__ chunk_counts) {
  __shared__ int cnt[MOE_MAX_E];
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * MOE_PERMUTE_CHUNK;
  const int end = min(base + MOE_PERMUTE_CHUNK, n);
  for (int i = base + threadIdx.x; i < end; i += 256) atomicAdd(&cnt[idx[i]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) chunk_counts[(size_t)blockIdx.x * E + e] = cnt[e];
}

// Turns chunk_counts[c][e] into the first row of chunk c's pairs of expert e.
// NREG > 0 (nchunk <= NREG): thread e holds its whole column in registers, so
// the column is read in one round of loads and written once; NREG == 0: any
// nchunk, 8 chunk rows at a time, read twice.
template <int NREG>
__global__ __launch_bounds__(1024) void permute_scan_kernel(int32_t* __restrict__ chunk_counts, int nchunk, int E,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets) {
  __shared__ int wsum[16];
  const int e = threadIdx.x;
  // 8 chunk rows at a time: their loads are issued before any store (the
  // compiler cannot tell that row c + 1 is not the word just stored)
  constexpr int NB = 8;
  int col[NREG > 0 ? NREG : 1];  // NREG > 0: exclusive prefix of the column
  int run = 0;
  if (e < E) {
    if constexpr (NREG > 0) {
#pragma unroll
      for (int c = 0; c < NREG; ++c) col[c] = c < nchunk ? chunk_counts[(size_t)c * E + e] : 0;
#pragma unroll
      for (int c = 0; c < NREG; ++c) {
        const int v = col[c];
        col[c] = run;
        run += v;
      }
    } else {
      for (int c0 = 0; c0 < nchunk; c0 += NB) {
        int v[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) v[j] = c0 + j < nchunk ? chunk_counts[(size_t)(c0 + j) * E + e] : 0;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if (c0 + j < nchunk) chunk_counts[(size_t)(c0 + j) * E + e] = run;
          run += v[j];
        }
      }
    }
  }
  // exclusive scan of the expert totals: within each wave (shuffles), then
  // over the 16 waves' totals (one barrier)
  const int lane = e & 63, wave = e >> 6;
  const int own = (e < E) ? run : 0;
  int incl = own;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  for (int w = 0; w < wave; ++w) incl += wsum[w];
  const int excl = incl - own;
  if (e < E) {
    counts[e] = run;
    offsets[e] = excl;
    if constexpr (NREG > 0) {
#pragma unroll
      for (int c = 0; c < NREG; ++c)
        if (c < nchunk) chunk_counts[(size_t)c * E + e] = col[c] + excl;
    } else {
      for (int c0 = 0; c0 < nchunk; c0 += NB) {
        int v[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) v[j] = c0 + j < nchunk ? chunk_counts[(size_t)(c0 + j) * E + e] : 0;
#pragma unroll
        for (int j = 0; j < NB; ++j)
          if (c0 + j < nchunk) chunk_counts[(size_t)(c0 + j) * E + e] = v[j] + excl;
      }
    }
  }
  if (e == E - 1) offsets[E] = incl;
}

// PS_WAVES waves per chunk: wave w walks pairs [128w, 128w + 128) of it, its
// running row of expert e starting at the chunk's base row of e plus the
// pairs of e in the parts before it (counted in LDS first); the rows come out
// in the same stable order as with one wave walking the whole chunk.
#define PS_WAVES 8
__global__ __launch_bounds__(64 * PS_WAVES) void permute_scatter_kernel(const int32_t* __restrict__ idx, int n,
                                                                        int E,
                                                                        const int32_t* __restrict__ chunk_base,
                                                                        int32_t* __restrict__ row_src,
                                                                        int32_t* __restrict__ inv_row) {
  __shared__ int run[PS_WAVES][MOE_MAX_E];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int PART = MOE_PERMUTE_CHUNK / PS_WAVES;
  static_assert(PART % 64 == 0, "a wave walks whole batches of 64 pairs");
  constexpr int NIT = PART / 64;
  const int base = blockIdx.x * MOE_PERMUTE_CHUNK + wave * PART;
  const int end = min(base + PART, n);  // <= base when this part is past n
  // this wave's expert ids, all requested before the first batch
  int ev[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int i = base + 64 * it + lane;
    ev[it] = i < end ? idx[i] : 0;
  }
#pragma unroll
  for (int w = 0; w < PS_WAVES; ++w)
    for (int e = tid; e < E; e += 64 * PS_WAVES) run[w][e] = 0;
  __syncthreads();
#pragma unroll
  for (int it = 0; it < NIT; ++it)
    if (base + 64 * it + lane < end) atomicAdd(&run[wave][ev[it]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += 64 * PS_WAVES) {
    int acc = chunk_base[(size_t)blockIdx.x * E + e];
#pragma unroll
    for (int w = 0; w < PS_WAVES; ++w) {
      const int c = run[w][e];
      run[w][e] = acc;
      acc += c;
    }
  }
  __syncthreads();
  // from here on each wave touches only its own run[wave]: no workgroup
  // barrier (the waves' batch counts differ in the last chunk)
  int* myrun = run[wave];
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int i0 = base + 64 * it;
    if (i0 >= end) break;
    const int i = i0 + lane;
    const bool valid = i < end;
    const int e = ev[it];
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lt_mask);
    const int r0 = valid ? myrun[e] : 0;
    __builtin_amdgcn_wave_barrier();  // every lane has read before the leaders write
    if (valid && rank == 0) myrun[e] = r0 + __popcll(peers);
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      const int row = r0 + rank;
      row_src[row] = i;
      inv_row[i] = row;
    }
  }
}

// x_perm[r] = x[row_src[r] / k], 16 bytes per thread.
__global__ __launch_bounds__(256) void permute_gather_kernel(const uint4* __restrict__ x, int k, int row_vec,
                                                             const int32_t* __restrict__ row_src,
                                                             uint4* __restrict__ x_perm) {
  const int r = blockIdx.x;
  const int t = row_src[r] / k;
  for (int v = threadIdx.x; v < row_vec; v += 256) x_perm[(size_t)r * row_vec + v] = x[(size_t)t * row_vec + v];
}

extern "C" int moe_permute(const int32_t* topk_idx, int T, int k, int E, int32_t* counts, int32_t* offsets,
                           int32_t* row_src, int32_t* inv_row, const void* x, int x_dtype, int H, void* x_perm,
                           void* ws, size_t ws_bytes, void* stream) {
  MOE_REQUIRE(T >= 0, MOE_ESHAPE, "T=%d must be >= 0", T);
  MOE_REQUIRE(E >= 1 && E <= MOE_MAX_E, MOE_ESHAPE, "E=%d out of [1, %d]", E, MOE_MAX_E);
  MOE_REQUIRE(k >= 1 && k <= MOE_MAX_K && k <= E, MOE_ESHAPE, "k=%d out of [1, min(E, %d)]", k, MOE_MAX_K);
  MOE_REQUIRE((int64_t)T * k < (1ll << 31), MOE_ESHAPE, "T*k must be < 2^31");
  MOE_REQUIRE(counts && offsets, MOE_EINVAL, "counts and offsets are required");
  MOE_REQUIRE(T == 0 || (topk_idx && row_src && inv_row), MOE_EINVAL, "topk_idx, row_src and inv_row are required");
  MOE_REQUIRE((x == nullptr) == (x_perm == nullptr), MOE_EINVAL, "x and x_perm must both be given or both be NULL");
  if (x_perm) {
    MOE_REQUIRE(x_dtype == MOE_F32 || x_dtype == MOE_BF16, MOE_EUNSUPPORTED, "x_dtype %d", x_dtype);
    MOE_REQUIRE(H >= 8 && H % 8 == 0 && H <= MOE_MAX_H, MOE_ESHAPE, "H=%d must be a multiple of 8", H);
    MOE_REQUIRE(moe_aligned(x, 16) && moe_aligned(x_perm, 16), MOE_EALIGN, "x and x_perm must be 16-byte aligned");
  }
  const int n = T * k;
  const int nchunk = moe_permute_nchunk(T, k);
  const size_t need = moe_ws_permute(T, k, E);
  MOE_REQUIRE(need == 0 || (ws && ws_bytes >= need), MOE_EWORKSPACE, "ws needs %zu bytes", need);
  hipStream_t st = moe_stream(stream);
  int32_t* cc = (int32_t*)ws;
  if (nchunk > 0) permute_hist_kernel<<<nchunk, 256, 0, st>>>(topk_idx, n, E, cc);
  if (nchunk <= 80)  // 80 column registers fit the 128 of a 1024-thread workgroup
    permute_scan_kernel<80><<<1, 1024, 0, st>>>(cc, nchunk, E, counts, offsets);
  else
    permute_scan_kernel<0><<<1, 1024, 0, st>>>(cc, nchunk, E, counts, offsets);
  if (nchunk > 0) permute_scatter_kernel<<<nchunk, 64 * PS_WAVES, 0, st>>>(topk_idx, n, E, cc, row_src, inv_row);
  if (x_perm && n > 0) {
    const int esize = x_dtype == MOE_F32 ? 4 : 2;
    permute_gather_kernel<<<n, 256, 0, st>>>((const uint4*)x, k, H * esize / 16, row_src, (uint4*)x_perm);
  }
  return moe_check_launch("permute");
}
