// Weighted sum of each token's expert outputs: the GPU adds up the chosen
// experts' results before the next layer starts ("为什么 Strata 在小显存显卡上
// 这么快", section "一个 token，三路工人").  Fixed order j = 0..k-1, then the
// shared expert (weight 1), then the residual; fp32; no atomics.
#include "moe_common.h"
#include "moe_kernels.h"

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_rows,
                                                      const int32_t* __restrict__ inv_row,
                                                      const float* __restrict__ y_shared,
                                                      const float* __restrict__ topk_w,
                                                      const float* residual, int k, int H,
                                                      float* y_out) {
  const int t = blockIdx.y;
  const int h = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (h >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float w = topk_w[(size_t)t * k + j];
    const size_t row = inv_row ? (size_t)inv_row[(size_t)t * k + j] : (size_t)t * (k + 1) + j;
    const float4 v = *reinterpret_cast<const float4*>(y_rows + row * H + h);
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  const float* sh = inv_row ? y_shared + (size_t)t * H : y_rows + ((size_t)t * (k + 1) + k) * H;
  const float4 s = *reinterpret_cast<const float4*>(sh + h);
  acc.x += s.x; acc.y += s.y; acc.z += s.z; acc.w += s.w;
  if (residual) {
    const float4 r = *reinterpret_cast<const float4*>(residual + (size_t)t * H + h);
    acc.x += r.x; acc.y += r.y; acc.z += r.z; acc.w += r.w;
  }
  *reinterpret_cast<float4*>(y_out + (size_t)t * H + h) = acc;
}

int moe_launch_combine(const float* y_rows, const int32_t* inv_row, const float* y_shared, const float* topk_w,
                       const float* residual, int T, int k, int H, float* y_out, hipStream_t st) {
  if (T == 0) return MOE_OK;
  dim3 grid((H / 4 + 255) / 256, T);
  combine_kernel<<<grid, 256, 0, st>>>(y_rows, inv_row, y_shared, topk_w, residual, k, H, y_out);
  return moe_check_launch("combine");
}

extern "C" int moe_combine(const float* y_rows, const int32_t* inv_row, const float* y_shared,
                           const float* topk_w, const float* residual, int T, int k, int H, float* y_out,
                           void* stream) {
  MOE_REQUIRE(T >= 0 && T < 65536 * 32, MOE_ESHAPE, "T=%d out of range", T);
  MOE_REQUIRE(k >= 1 && k <= MOE_MAX_K, MOE_ESHAPE, "k=%d out of [1, %d]", k, MOE_MAX_K);
  MOE_REQUIRE(H >= 4 && H % 4 == 0 && H <= MOE_MAX_H, MOE_ESHAPE, "H=%d must be a multiple of 4", H);
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(y_rows && topk_w && y_out, MOE_EINVAL, "y_rows, topk_w and y_out are required");
  MOE_REQUIRE((inv_row == nullptr) == (y_shared == nullptr), MOE_EINVAL,
              "inv_row and y_shared are given together (prefill layout) or both NULL (decode layout)");
  MOE_REQUIRE(moe_aligned(y_rows, 16) && moe_aligned(y_out, 16) && (!residual || moe_aligned(residual, 16)) &&
                  (!y_shared || moe_aligned(y_shared, 16)),
              MOE_EALIGN, "y_rows, y_shared, residual and y_out must be 16-byte aligned");
  return moe_launch_combine(y_rows, inv_row, y_shared, topk_w, residual, T, k, H, y_out, moe_stream(stream));
}
