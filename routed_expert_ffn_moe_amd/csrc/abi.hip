// Housekeeping entry points of libmoe: version, errors, sizes.
#include <cstdarg>
#include <cstdio>

#include "moe_common.h"
#include "moe_sizes.h"
#include "moe_kernels.h"

static thread_local char g_err[512] = "";

int moe_fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int moe_check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return moe_fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

int moe_check_expert_shapes(int H, int F, int E, int k, int qfmt, const void* pool,
                            int64_t record_bytes, const int32_t* slot_table, int layer) {
  MOE_REQUIRE(qfmt == MOE_Q4_B32 || qfmt == MOE_Q2_B16, MOE_EUNSUPPORTED, "unknown qfmt %d", qfmt);
  MOE_REQUIRE(H >= 128 && H <= MOE_MAX_H && H % 128 == 0, MOE_ESHAPE, "H=%d must be a multiple of 128 in [128, %d]", H, MOE_MAX_H);
  MOE_REQUIRE(F >= 128 && F <= MOE_MAX_F && F % 128 == 0, MOE_ESHAPE, "F=%d must be a multiple of 128 in [128, %d]", F, MOE_MAX_F);
  MOE_REQUIRE(E >= 1 && E <= MOE_MAX_E, MOE_ESHAPE, "E=%d out of [1, %d]", E, MOE_MAX_E);
  MOE_REQUIRE(k >= 1 && k <= MOE_MAX_K && k <= E, MOE_ESHAPE, "k=%d out of [1, min(E, %d)]", k, MOE_MAX_K);
  MOE_REQUIRE(pool != nullptr && slot_table != nullptr, MOE_EINVAL, "pool and slot_table are required");
  MOE_REQUIRE(moe_aligned(pool, 256), MOE_EALIGN, "pool must be 256-byte aligned");
  MOE_REQUIRE(record_bytes % 256 == 0 && record_bytes >= moe_record_bytes(qfmt, H, F), MOE_EALIGN,
              "record_bytes=%lld must be a multiple of 256 and >= %lld", (long long)record_bytes,
              (long long)moe_record_bytes(qfmt, H, F));
  MOE_REQUIRE(layer >= 0, MOE_EINVAL, "layer=%d must be >= 0", layer);
  return MOE_OK;
}

extern "C" int moe_abi_version(void) { return MOE_ABI_VERSION; }

extern "C" const char* moe_last_error(void) { return g_err; }

extern "C" int64_t moe_record_bytes(int qfmt, int H, int F) {
  if (H < 128 || F < 128 || H % 128 || F % 128 || H > MOE_MAX_H || F > MOE_MAX_F) return 0;
  int64_t HF = (int64_t)H * F;
  if (qfmt == MOE_Q4_B32) return 27 * HF / 16;
  if (qfmt == MOE_Q2_B16) return 3 * HF / 2;
  return 0;
}

extern "C" size_t moe_workspace_size(int op, int T, int k, int E, int H, int F, int qfmt) {
  if (T < 0 || k < 0 || E < 0 || H < 0 || F < 0) return 0;
  switch (op) {
    case MOE_OP_ROUTE_TOPK: return moe_ws_route(T, E);
    case MOE_OP_PERMUTE: return moe_ws_permute(T, k, E);
    case MOE_OP_EXPERT_GEMV_Q: return moe_ws_gemv(T, k, H, F, qfmt);
    case MOE_OP_GROUPED_GEMM_Q: return moe_ws_gemm(T, k, E, H, F);
    case MOE_OP_COMBINE: return 0;
    case MOE_OP_USAGE_UPDATE: return 0;
    case MOE_OP_DECODE_STACK: return moe_ws_decode_stack(T, k, E, H, F, qfmt);
    default: return 0;
  }
}
