// Per-step expert usage with exponential decay and a periodic global re-rank.
// The more an expert is used, the harder it is to evict, by an exponentially
// decayed usage score ("Strata：12GB 显卡跑 125B 模型，MoE 专家热缓存打破 VRAM
// 限制", section "工作原理"); the adaptive tier swaps in at most 96 experts
// every four rounds ("为什么 Strata 在小显存显卡上这么快", section "由粗到细").
//
// decay pass: hits counted with LDS integer atomics (order-free), then
//   s = fl(fl(decay * s) + hits) with separately rounded multiply and add.
// re-rank: 64-bit keys (order-preserving score bits << 32 | ~flat index) are
//   unique; an 8-pass MSB radix select finds the top_n-th largest key, the
//   keys at or above it are gathered and bitonic-sorted (descending).
#include "moe_common.h"
#include "moe_select.h"

// Workgroup b updates layer layer0 + b from its routing idx[b][T][k] (hits in
// hits_ws[b][E]): one launch per layer, or one for a whole stack.
__global__ __launch_bounds__(1024) void usage_decay_kernel(const int32_t* __restrict__ idx, int T, int k, int layer0,
                                                           int E, float decay, int32_t* __restrict__ hits_ws,
                                                           float* __restrict__ scores) {
  __shared__ int hits[MOE_MAX_E];
  const int layer = layer0 + (int)blockIdx.x;
  idx += (size_t)blockIdx.x * T * k;
  hits_ws += (size_t)blockIdx.x * E;
  for (int e = threadIdx.x; e < E; e += 1024) hits[e] = 0;
  __syncthreads();
  const int n = T * k;
  for (int i = threadIdx.x; i < n; i += 1024) {
    const int t = i / k, j = i - t * k;
    const int e = idx[i];
    bool first = true;
    for (int jj = 0; jj < j; ++jj) first &= idx[t * k + jj] != e;
    if (first) atomicAdd(&hits[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 1024) {
    // separately rounded multiply and add: no contraction into an FMA
#pragma clang fp contract(off)
    hits_ws[e] = hits[e];
    float* s = scores + (size_t)layer * E + e;
    const float d = decay * *s;
    *s = d + (float)hits[e];
  }
}

__device__ __forceinline__ uint64_t usage_key(const float* s, int i) {
  return ((uint64_t)moe_f32_order_key(s[i]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)i);
}

__global__ __launch_bounds__(1024) void usage_rerank_kernel(const float* __restrict__ scores, int N, int top_n,
                                                            int32_t* __restrict__ top_out) {
  __shared__ uint64_t sel[1024];
  moe_top_keys_sorted([&](int i) { return usage_key(scores, i); }, N, top_n, sel);
  if (threadIdx.x < top_n) top_out[threadIdx.x] = (int32_t)(0xFFFFFFFFu - (uint32_t)sel[threadIdx.x]);
}

extern "C" int moe_usage_update_stack(const int32_t* topk_idx, int T, int k, int L, int E, float decay, int64_t step,
                                      int rerank_every, int top_n, int32_t* hits_ws, float* scores, int32_t* top_out,
                                      void* stream) {
  MOE_REQUIRE(T >= 0 && (int64_t)T * k * L < (1ll << 31), MOE_ESHAPE, "T=%d out of range", T);
  MOE_REQUIRE(E >= 1 && E <= MOE_MAX_E, MOE_ESHAPE, "E=%d out of [1, %d]", E, MOE_MAX_E);
  MOE_REQUIRE(k >= 1 && k <= MOE_MAX_K && k <= E, MOE_ESHAPE, "k=%d out of [1, min(E, %d)]", k, MOE_MAX_K);
  MOE_REQUIRE(L >= 1 && (int64_t)L * E <= 65536, MOE_ESHAPE, "L*E must be in [1, 65536]");
  MOE_REQUIRE(rerank_every >= 1 && step >= 0, MOE_EINVAL, "rerank_every must be >= 1 and step >= 0");
  MOE_REQUIRE(top_n >= 1 && top_n <= 1024 && top_n <= L * E, MOE_ESHAPE, "top_n=%d out of [1, min(L*E, 1024)]", top_n);
  MOE_REQUIRE(__builtin_isfinite(decay) && decay >= 0.f, MOE_EINVAL, "decay must be finite and >= 0");
  MOE_REQUIRE(hits_ws && scores && (T == 0 || topk_idx), MOE_EINVAL, "hits_ws, scores and topk_idx are required");
  hipStream_t st = moe_stream(stream);
  usage_decay_kernel<<<L, 1024, 0, st>>>(topk_idx, T, k, 0, E, decay, hits_ws, scores);
  if (top_out && (step + 1) % rerank_every == 0)
    usage_rerank_kernel<<<1, 1024, 0, st>>>(scores, L * E, top_n, top_out);
  return moe_check_launch("usage update (stack)");
}

extern "C" int moe_usage_update(const int32_t* topk_idx, int T, int k, int layer, int L, int E, float decay,
                                int64_t step, int rerank_every, int top_n, int32_t* hits_ws, float* scores,
                                int32_t* top_out, void* stream) {
  MOE_REQUIRE(T >= 0 && (int64_t)T * k < (1ll << 31), MOE_ESHAPE, "T=%d out of range", T);
  MOE_REQUIRE(E >= 1 && E <= MOE_MAX_E, MOE_ESHAPE, "E=%d out of [1, %d]", E, MOE_MAX_E);
  MOE_REQUIRE(k >= 1 && k <= MOE_MAX_K && k <= E, MOE_ESHAPE, "k=%d out of [1, min(E, %d)]", k, MOE_MAX_K);
  MOE_REQUIRE(L >= 1 && (int64_t)L * E <= 65536, MOE_ESHAPE, "L*E must be in [1, 65536]");
  MOE_REQUIRE(layer >= 0 && layer < L, MOE_EINVAL, "layer=%d out of [0, L)", layer);
  MOE_REQUIRE(rerank_every >= 1 && step >= 0, MOE_EINVAL, "rerank_every must be >= 1 and step >= 0");
  MOE_REQUIRE(top_n >= 1 && top_n <= 1024 && top_n <= L * E, MOE_ESHAPE, "top_n=%d out of [1, min(L*E, 1024)]", top_n);
  MOE_REQUIRE(__builtin_isfinite(decay) && decay >= 0.f, MOE_EINVAL, "decay must be finite and >= 0");
  MOE_REQUIRE(hits_ws && scores && (T == 0 || topk_idx), MOE_EINVAL, "hits_ws, scores and topk_idx are required");
  hipStream_t st = moe_stream(stream);
  usage_decay_kernel<<<1, 1024, 0, st>>>(topk_idx, T, k, layer, E, decay, hits_ws, scores);
  if (top_out && layer == L - 1 && (step + 1) % rerank_every == 0)
    usage_rerank_kernel<<<1, 1024, 0, st>>>(scores, L * E, top_n, top_out);
  return moe_check_launch("usage update");
}
