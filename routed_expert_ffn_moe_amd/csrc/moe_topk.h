// Top-k selection of one token's router logits by one wave: the choice
// rule is the router's (the k largest fp32 logits, larger first, equal
// logits to the lower expert index; the weights are the softmax of the
// chosen logits), as in "Strata开源运行时：12GB显卡跑动125B参数Qwen3模型",
// section "模型本身：稀疏MoE带来的计算与存储鸿沟".  Used by the decode kernel
// (one token per wave inside the layer loop) and by the top-k kernel of the
// separate router path.
#pragma once
#include "moe_common.h"

// The lane index, made opaque at each call (values derived from it are
// computed where used instead of being kept live across a long kernel).
__device__ __forceinline__ int moe_topk_lane() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t & 63;
}

// wave-wide max of uint32 entirely in DPP (row_bcast15 / row_bcast31 carry the
// row maxima upwards), read from lane 63
__device__ __forceinline__ uint32_t moe_wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast31
  return __builtin_amdgcn_readlane(v, 63);
}

// Top-k by repeated extraction (the fallback of moe_topk_select below): each lane
// sorts its keys; every round takes the wave-wide maximum of the lane heads
// and the lane holding it pops its head.  Lane j < k ends with the j-th key
// and expert.
template <int SLOTS>
__device__ __forceinline__ void moe_topk_rounds(uint32_t (&hi)[SLOTS], int k, uint32_t& my_key, uint32_t& my_e) {
  const int lane = moe_topk_lane();
  uint32_t ex[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) ex[i] = (uint32_t)(lane + 64 * i);
  // descending sort of the lane's keys (odd-even transposition network); the
  // experts of one lane ascend with i, so equal keys keep the lower expert first
#pragma unroll
  for (int r = 0; r < SLOTS; ++r) {
#pragma unroll
    for (int i = r & 1; i + 1 < SLOTS; i += 2) {
      const bool sw = hi[i] < hi[i + 1] || (hi[i] == hi[i + 1] && ex[i] > ex[i + 1]);
      const uint32_t h0 = hi[i], e0 = ex[i];
      hi[i] = sw ? hi[i + 1] : hi[i];
      ex[i] = sw ? ex[i + 1] : ex[i];
      hi[i + 1] = sw ? h0 : hi[i + 1];
      ex[i + 1] = sw ? e0 : ex[i + 1];
    }
  }
  int pos = 0;  // the lane's head is entry `pos` of its sorted keys (past the end: key 0)
  uint32_t head = hi[0], head_e = ex[0];
  for (int j = 0; j < k; ++j) {
    const uint32_t M = moe_wave_max_u32(head);
    const uint64_t cand = __ballot(head == M);
    int wl = __ffsll((long long)cand) - 1;
    if (__popcll(cand) > 1) {  // equal logits in several lanes: the lowest expert
      const uint32_t ce = head == M ? head_e : 0xFFFFFFFFu;
      const uint32_t emin = ~moe_wave_max_u32(~ce);
      wl = (int)(emin & 63);
    }
    const uint32_t ew = __builtin_amdgcn_readlane(head_e, wl);
    my_key = lane == j ? M : my_key;
    my_e = lane == j ? ew : my_e;
    pos += lane == wl;
    uint32_t nh = 0u, ne = 0u;
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      nh = pos == i ? hi[i] : nh;
      ne = pos == i ? ex[i] : ne;
    }
    head = nh;
    head_e = ne;
  }
}

// Top-k of one token's E <= 64 * SLOTS logits (LDS or global memory) by one wave.  Lane l holds the keys of
// experts l + 64 * i (i < SLOTS): the order-preserving bits of the logit; the
// order is by key, and on equal keys the lower expert first.
//  1. tau = the k-th largest lane maximum, its top 16 bits found with ballots
//     (the rest left 0): at least k keys are >= tau, so every chosen
//     expert's key is >= tau.
//  2. The keys >= tau (usually a few more than k) are packed into `cand` as
//     key << 32 | ~expert, which orders them exactly as the rule above.
//  3. Each candidate's rank = the number of larger candidates; rank j < k is
//     the j-th choice.
// More than 64 candidates (many equal logits) take the extraction rounds.
// Lane j < k writes the j-th expert to ids[j] and returns its key (the
// weights follow in moe_topk_weights).  `cand`: 64 words of LDS for this wave.
template <int SLOTS>
__device__ __forceinline__ uint32_t moe_topk_select(const float* lg, int E, int k, int* ids, uint64_t* cand) {
  const int lane = moe_topk_lane();
  uint32_t hi[SLOTS];
  uint32_t head = 0u;
  float v[SLOTS];  // every load is issued before the first use
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) v[i] = lg[min(lane + 64 * i, E - 1)];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const uint32_t key = moe_f32_order_key(v[i]);
    hi[i] = lane + 64 * i < E ? key : 0u;  // every real key is > 0
    head = max(head, hi[i]);
  }
  // one bit per step, bits 31..16; the low 16 bits stay 0, which only lowers
  // tau (keys within about 1% of the k-th lane maximum join the candidates)
  uint32_t tau = 0u;
#pragma unroll
  for (int b = 31; b >= 16; --b) {
    const uint32_t c = tau | (1u << b);
    tau = __popcll(__ballot(head >= c)) >= k ? c : tau;
  }
  int n = 0;
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const bool t = hi[i] >= tau && lane + 64 * i < E;
    const uint64_t m = __ballot(t);
    const int p = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (t && p < 64) cand[p] = ((uint64_t)hi[i] << 32) | (uint32_t)~(uint32_t)(lane + 64 * i);
    n += __popcll(m);
  }
  uint32_t my_key = 0u, my_e = 0u;
  if (n <= 64) {
    const int n8 = (n + 7) & ~7;
    if (lane >= n && lane < n8) cand[lane] = 0ull;  // pads: below every candidate
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const uint64_t me = cand[lane];
    int rank = 0;
    for (int m = 0; m < n8; m += 8) {
#pragma unroll
      for (int q = 0; q < 8; ++q) rank += cand[m + q] > me;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (lane < n && rank < k) cand[rank] = me;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const uint64_t w = cand[lane < k ? lane : 0];
    my_key = lane < k ? (uint32_t)(w >> 32) : 0u;
    my_e = lane < k ? ~(uint32_t)w : 0u;
  } else {
    moe_topk_rounds<SLOTS>(hi, k, my_key, my_e);
  }
  if (lane < k) ids[lane] = (int)my_e;
  return my_key;
}

// Softmax weights of the chosen logits, lane j < k holding the key of the
// j-th (the largest in lane 0): wts[j].  One wave.
__device__ __forceinline__ void moe_topk_weights(uint32_t my_key, int k, float* wts) {
  const int lane = moe_topk_lane();
  const float m0 = moe_order_key_f32(__builtin_amdgcn_readfirstlane(my_key));
  const float z = lane < k ? expf(moe_order_key_f32(my_key) - m0) : 0.f;
  float sum = z;  // sum in lane order: lanes 0..k-1 are added left to right
  {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), j));
    sum = acc;
  }
  if (lane < k) wts[lane] = z / sum;
}
