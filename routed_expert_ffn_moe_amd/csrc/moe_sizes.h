// Workspace layouts of the entry points.  The size query and the entry points
// both use these functions, so they always agree.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

#define MOE_WS_ALIGN 256
#define MOE_PERMUTE_CHUNK 1024  // (token, choice) pairs per permutation block
#define MOE_GEMM_BM 128         // rows per grouped-GEMM tile

static inline size_t moe_ws_up(size_t v) { return (v + MOE_WS_ALIGN - 1) / MOE_WS_ALIGN * MOE_WS_ALIGN; }

// ---- route_topk: logits [T][E] fp32
static inline size_t moe_ws_route(int T, int E) { return moe_ws_up((size_t)T * E * 4); }

// ---- permute: per-chunk expert counts [nchunk][E] int32
static inline int moe_permute_nchunk(int T, int k) {
  return (int)(((int64_t)T * k + MOE_PERMUTE_CHUNK - 1) / MOE_PERMUTE_CHUNK);
}
static inline size_t moe_ws_permute(int T, int k, int E) {
  return moe_ws_up((size_t)moe_permute_nchunk(T, k) * E * 4);
}

// ---- expert_gemv_q
// plan: U, then per unique expert u < UMAX: expert id, token count, tokens,
// choice positions.  Prepared activations ("prep"): per vector of K values,
// K fp16 (pairs ordered for the dot2 inner loop) followed by one float2
// correction per quantisation block.
struct MoeGemvLayout {
  int umax;
  size_t plan, xprep, hprep, total;
  size_t xprep_stride, hprep_stride;  // bytes per prepared vector
};
static inline int moe_qblock(int qfmt) { return qfmt == MOE_Q4_B32 ? 32 : 16; }
static inline size_t moe_prep_bytes(int K, int qfmt) {
  return moe_ws_up((size_t)K * 2 + (size_t)(K / moe_qblock(qfmt)) * 8);
}
static inline MoeGemvLayout moe_gemv_layout(int T, int k, int H, int F, int qfmt) {
  MoeGemvLayout L;
  L.umax = T * k + 1;
  size_t plan_ints = 1 + (size_t)L.umax * (2 + 2 * (size_t)MOE_MAX_DECODE_T);
  L.xprep_stride = moe_prep_bytes(H, qfmt);
  L.hprep_stride = moe_prep_bytes(F, qfmt);
  L.plan = 0;
  L.xprep = moe_ws_up(plan_ints * 4);
  L.hprep = L.xprep + L.xprep_stride * (size_t)T;
  // prepared h of (distinct expert u, its i-th token) at (u * MOE_MAX_DECODE_T + i)
  L.total = L.hprep + L.hprep_stride * (size_t)L.umax * MOE_MAX_DECODE_T;
  return L;
}
static inline size_t moe_ws_gemv(int T, int k, int H, int F, int qfmt) {
  if (T < 1 || k < 1 || H < 128 || F < 128) return 0;
  return moe_gemv_layout(T, k, H, F, qfmt).total;
}

// ---- grouped_gemm_q: tile starts [E+2] int32, then h fp16 [T*k + T][F]
static inline int moe_gemm_max_tiles(int T, int k, int E) {
  return (int)(((int64_t)T * k) / MOE_GEMM_BM + E + ((int64_t)T + MOE_GEMM_BM - 1) / MOE_GEMM_BM + 1);
}
// grouped GEMM workspace: tile_start [E+2] int32, tile_info [max_tiles] int4,
static inline size_t moe_gemm_info_offset(int E) { return moe_ws_up((size_t)(E + 2) * 4); }
static inline size_t moe_gemm_h_offset(int T, int k, int E) {
  return moe_gemm_info_offset(E) + moe_ws_up((size_t)moe_gemm_max_tiles(T, k, E) * 16);
}
// then h (fp16) [T*k + T][F], then x converted to fp16 [T][H]
static inline size_t moe_gemm_x16_offset(int T, int k, int E, int F) {
  return moe_gemm_h_offset(T, k, E) + moe_ws_up(((size_t)T * k + T) * F * 2);
}
static inline size_t moe_ws_gemm(int T, int k, int E, int H, int F) {
  return moe_gemm_x16_offset(T, k, E, F) + moe_ws_up((size_t)T * H * 2);
}

// ---- decode_stack: per-layer scratch reused across layers
struct MoeStackLayout {
  size_t xn, logits, idx, w, yparts, gemv, total;
};
static inline MoeStackLayout moe_stack_layout(int T, int k, int E, int H, int F, int qfmt) {
  MoeStackLayout L;
  L.xn = 0;
  L.logits = L.xn + moe_ws_up((size_t)T * H * 4);
  L.idx = L.logits + moe_ws_up((size_t)T * E * 4);
  L.w = L.idx + moe_ws_up((size_t)T * k * 4);
  L.yparts = L.w + moe_ws_up((size_t)T * k * 4);
  L.gemv = L.yparts + moe_ws_up((size_t)T * (k + 1) * H * 4);
  L.total = L.gemv + moe_ws_gemv(T, k, H, F, qfmt);
  return L;
}
static inline size_t moe_ws_stack(int T, int k, int E, int H, int F, int qfmt) {
  if (T < 1 || k < 1) return 0;
  return moe_stack_layout(T, k, E, H, F, qfmt).total;
}
