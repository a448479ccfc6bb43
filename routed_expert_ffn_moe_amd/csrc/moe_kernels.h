// Internal launchers shared between the entry points (not part of the ABI).
#pragma once
#include "moe_common.h"

int moe_launch_route(const void* x, int x_dtype, int T, int H, const uint16_t* w_router, const float* bias,
                     int E, int k, int32_t* topk_idx, float* topk_w, float* logits, hipStream_t st);

int moe_launch_gemv(const float* x, int T, int H, int F, const int32_t* topk_idx, int k, int E,
                    const int32_t* slot_table, int layer, const void* pool, int64_t record_bytes, int qfmt,
                    float* y_parts, void* ws, hipStream_t st);

int moe_launch_combine(const void* y_rows, int rows_dtype, const int32_t* inv_row, const void* y_shared,
                       const float* topk_w, const float* residual, int T, int k, int H, float* y_out, hipStream_t st);

// Persistent single-kernel decode step (decode_persistent.hip).
size_t moe_ws_stack_persistent(int T, int k, int E, int H, int F, int qfmt);
bool moe_persistent_supported(int T, int k, int E, int H, int F, int qfmt);
bool moe_persistent_coresident(int T, int k, int E, int H, int F, int qfmt);
int moe_launch_decode_persistent(const float* x_in, int T, int H, int F, int E, int k, int L,
                                 const uint16_t* w_router, const float* bias, const int32_t* slot_table,
                                 const void* pool, int64_t record_bytes, int qfmt, float* x_out,
                                 int32_t* topk_idx_out, float* topk_w_out, float* x_hist, void* ws,
                                 size_t ws_bytes, hipStream_t st);

// Workspace of moe_decode_stack: enough for whichever path it takes.
size_t moe_ws_decode_stack(int T, int k, int E, int H, int F, int qfmt);

// moe_decode_stack's argument checks (everything but the workspace) and its
// body once the workspace is known to be large enough.
int moe_decode_stack_check(const float* x_in, int T, int H, int F, int E, int k, int L, const uint16_t* w_router,
                           const int32_t* slot_table, const void* pool, int64_t record_bytes, int qfmt,
                           const float* x_out, const float* x_hist);
int moe_decode_stack_run(const float* x_in, int T, int H, int F, int E, int k, int L, const uint16_t* w_router,
                         const float* bias, const int32_t* slot_table, const void* pool, int64_t record_bytes,
                         int qfmt, float* x_out, int32_t* topk_idx_out, float* topk_w_out, float* x_hist, void* ws,
                         size_t ws_bytes, hipStream_t st);

// The stack's pre-norm (rmsnorm.hip), fp32 or bf16 output.
int moe_launch_rmsnorm(const float* x, int T, int H, float eps, void* out, int out_dtype, hipStream_t st);
