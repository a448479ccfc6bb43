// One decode / verify step through L chained MoE layers.
// Every token passes through all 48 layers in order ("Strata开源运行时：12GB显卡
// 跑动125B参数Qwen3模型", section "推测解码：用模型自身的草稿层加速生成"); the
// engine records the whole forward once and replays it so the host never waits
// inside a step ("为什么 Strata 在小显存显卡上这么快", section "一个 token，三路
// 工人").  Here the step is enqueued as one chain on the caller's stream (and
// can be captured into a HIP graph by the caller).  Per layer:
//   xn = x / sqrt(mean(x^2) + 1e-6)      (pre-norm, unit gain)
//   router + top-k on xn, expert GEMV on xn, x <- x + combine.
// The pages do not describe the non-MoE parts of a layer; without the norm a
// chain of SwiGLU layers (quadratic in x) overflows within a few layers.
#include "moe_common.h"
#include "moe_sizes.h"
#include "moe_kernels.h"

#include <cstdlib>
#include <cstring>

#define MOE_STACK_EPS 1e-6f

size_t moe_ws_decode_stack(int T, int k, int E, int H, int F, int qfmt) {
  if (T < 1 || k < 1 || H < 128 || F < 128) return 0;
  size_t a = moe_ws_stack(T, k, E, H, F, qfmt);
  if (moe_persistent_supported(T, k, E, H, F, qfmt)) {
    const size_t b = moe_ws_stack_persistent(T, k, E, H, F, qfmt);
    if (b > a) a = b;
  }
  return a;
}

// MOE_DECODE_PATH=chain forces the per-layer kernel chain; otherwise the
// persistent kernel is used whenever it supports the shape and the device
// can keep all of its workgroups resident at once.
static bool use_persistent(int T, int k, int E, int H, int F, int qfmt) {
  const char* e = getenv("MOE_DECODE_PATH");
  if (e && strcmp(e, "chain") == 0) return false;
  return moe_persistent_supported(T, k, E, H, F, qfmt) && moe_persistent_coresident(T, k, E, H, F, qfmt);
}

int moe_decode_stack_check(const float* x_in, int T, int H, int F, int E, int k, int L, const uint16_t* w_router,
                           const int32_t* slot_table, const void* pool, int64_t record_bytes, int qfmt,
                           const float* x_out, const float* x_hist) {
  int rc = moe_check_expert_shapes(H, F, E, k, qfmt, pool, record_bytes, slot_table, 0);
  if (rc) return rc;
  MOE_REQUIRE(T >= 1 && T <= MOE_MAX_DECODE_T, MOE_ESHAPE, "T=%d out of [1, %d]", T, MOE_MAX_DECODE_T);
  MOE_REQUIRE(L >= 1, MOE_ESHAPE, "L=%d must be >= 1", L);
  MOE_REQUIRE(x_in && x_out && w_router, MOE_EINVAL, "x_in, x_out and w_router are required");
  MOE_REQUIRE(x_in != x_out, MOE_EINVAL, "x_out may not alias x_in");
  MOE_REQUIRE(moe_aligned(x_in, 16) && moe_aligned(x_out, 16) && moe_aligned(w_router, 16) &&
                  (!x_hist || moe_aligned(x_hist, 16)),
              MOE_EALIGN, "x_in, x_out, x_hist and w_router must be 16-byte aligned");
  return MOE_OK;
}

extern "C" int moe_decode_stack(const float* x_in, int T, int H, int F, int E, int k, int L,
                                const uint16_t* w_router, const float* bias, const int32_t* slot_table,
                                const void* pool, int64_t record_bytes, int qfmt, float* x_out,
                                int32_t* topk_idx_out, float* topk_w_out, float* x_hist, void* ws, size_t ws_bytes,
                                void* stream) {
  int rc = moe_decode_stack_check(x_in, T, H, F, E, k, L, w_router, slot_table, pool, record_bytes, qfmt, x_out,
                                  x_hist);
  if (rc) return rc;
  const size_t need = moe_ws_decode_stack(T, k, E, H, F, qfmt);
  MOE_REQUIRE(ws && ws_bytes >= need && moe_aligned(ws, 256), MOE_EWORKSPACE,
              "ws needs %zu bytes, 256-byte aligned", need);
  return moe_decode_stack_run(x_in, T, H, F, E, k, L, w_router, bias, slot_table, pool, record_bytes, qfmt, x_out,
                              topk_idx_out, topk_w_out, x_hist, ws, ws_bytes, moe_stream(stream));
}

int moe_decode_stack_run(const float* x_in, int T, int H, int F, int E, int k, int L, const uint16_t* w_router,
                         const float* bias, const int32_t* slot_table, const void* pool, int64_t record_bytes,
                         int qfmt, float* x_out, int32_t* topk_idx_out, float* topk_w_out, float* x_hist, void* ws,
                         size_t ws_bytes, hipStream_t st) {
  int rc = MOE_OK;
  if (use_persistent(T, k, E, H, F, qfmt))
    return moe_launch_decode_persistent(x_in, T, H, F, E, k, L, w_router, bias, slot_table, pool, record_bytes, qfmt,
                                        x_out, topk_idx_out, topk_w_out, x_hist, ws, ws_bytes, st);
  const MoeStackLayout W = moe_stack_layout(T, k, E, H, F, qfmt);
  uint8_t* w = (uint8_t*)ws;
  float* logits = (float*)(w + W.logits);
  float* yparts = (float*)(w + W.yparts);
  float* xn = (float*)(w + W.xn);
  void* gws = w + W.gemv;
  const size_t xbytes = (size_t)T * H * 4;
  if (hipMemcpyAsync(x_out, x_in, xbytes, hipMemcpyDeviceToDevice, st) != hipSuccess)
    return moe_fail(MOE_EHIP, "decode stack: copy of x_in failed");
  for (int l = 0; l < L; ++l) {
    int32_t* idx = topk_idx_out ? topk_idx_out + (size_t)l * T * k : (int32_t*)(w + W.idx);
    float* wt = topk_w_out ? topk_w_out + (size_t)l * T * k : (float*)(w + W.w);
    if (x_hist && hipMemcpyAsync(x_hist + (size_t)l * T * H, x_out, xbytes, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return moe_fail(MOE_EHIP, "decode stack: copy to x_hist failed");
    rc = moe_launch_rmsnorm(x_out, T, H, MOE_STACK_EPS, xn, MOE_F32, st);
    if (rc) return rc;
    rc = moe_launch_route(xn, MOE_F32, T, H, w_router + (size_t)l * E * H, bias ? bias + (size_t)l * E : nullptr,
                          E, k, idx, wt, logits, st);
    if (rc) return rc;
    rc = moe_launch_gemv(xn, T, H, F, idx, k, E, slot_table, l, pool, record_bytes, qfmt, yparts, gws, st);
    if (rc) return rc;
    rc = moe_launch_combine(yparts, MOE_F32, nullptr, nullptr, wt, x_out, T, k, H, x_out, st);
    if (rc) return rc;
  }
  return MOE_OK;
}
