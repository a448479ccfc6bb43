// Weighted sum of each token's expert outputs: the GPU adds up the chosen
// experts' results before the next layer starts ("为什么 Strata 在小显存显卡上
// 这么快", section "一个 token，三路工人").  Fixed order j = 0..k-1, then the
// shared expert (weight 1), then the residual; fp32 sums; no atomics.  The
// expert rows are fp32, or fp16 as the prefill grouped GEMM writes them.
#include "moe_common.h"
#include "moe_kernels.h"

typedef float moe_f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 moe_f16x4 __attribute__((ext_vector_type(4)));

// 4 consecutive values of a row as fp32; each expert row is read once
// (nontemporal: 20% faster at 8,192 tokens).
__device__ __forceinline__ float4 combine_ld4(const float* p) {
  const moe_f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const moe_f32x4*>(p));
  return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ float4 combine_ld4(const _Float16* p) {
  const moe_f16x4 t = __builtin_nontemporal_load(reinterpret_cast<const moe_f16x4*>(p));
  return make_float4((float)t.x, (float)t.y, (float)t.z, (float)t.w);
}

// KC > 0: k == KC at compile time, so that a thread requests all of its rows
// before the first add; KC == 0: any k, one row after another.  R: the type
// of the expert rows and of the shared rows.
template <int KC, typename R>
__global__ __launch_bounds__(256) void combine_kernel(const R* __restrict__ y_rows,
                                                      const int32_t* __restrict__ inv_row,
                                                      const R* __restrict__ y_shared,
                                                      const float* __restrict__ topk_w,
                                                      const float* residual, int k_rt, int H,
                                                      float* y_out) {
  const int k = KC > 0 ? KC : k_rt;
  const int t = blockIdx.y;
  const int h = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (h >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto row_of = [&](int j) {
    return inv_row ? (size_t)inv_row[(size_t)t * k + j] : (size_t)t * (k + 1) + j;
  };
  auto add = [&](int j, float4 v) {
    const float w = topk_w[(size_t)t * k + j];
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  };
  if constexpr (KC > 0) {
    size_t row[KC];
    if (inv_row) {
#pragma unroll
      for (int j = 0; j < KC; ++j) row[j] = (size_t)inv_row[(size_t)t * KC + j];
    } else {
#pragma unroll
      for (int j = 0; j < KC; ++j) row[j] = (size_t)t * (KC + 1) + j;
    }
    float4 v[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) v[j] = combine_ld4(y_rows + row[j] * H + h);
#pragma unroll
    for (int j = 0; j < KC; ++j) add(j, v[j]);
  } else {
    for (int j = 0; j < k; ++j) add(j, combine_ld4(y_rows + row_of(j) * H + h));
  }
  const R* sh = inv_row ? y_shared + (size_t)t * H : y_rows + ((size_t)t * (k + 1) + k) * H;
  const float4 s = combine_ld4(sh + h);
  acc.x += s.x; acc.y += s.y; acc.z += s.z; acc.w += s.w;
  if (residual) {
    const float4 r = *reinterpret_cast<const float4*>(residual + (size_t)t * H + h);
    acc.x += r.x; acc.y += r.y; acc.z += r.z; acc.w += r.w;
  }
  *reinterpret_cast<float4*>(y_out + (size_t)t * H + h) = acc;
}

template <typename R>
static void launch_combine_t(const R* y_rows, const int32_t* inv_row, const R* y_shared, const float* topk_w,
                             const float* residual, int T, int k, int H, float* y_out, hipStream_t st) {
  dim3 grid((H / 4 + 255) / 256, T);
  switch (k) {
    case 2: combine_kernel<2, R><<<grid, 256, 0, st>>>(y_rows, inv_row, y_shared, topk_w, residual, k, H, y_out); break;
    case 6: combine_kernel<6, R><<<grid, 256, 0, st>>>(y_rows, inv_row, y_shared, topk_w, residual, k, H, y_out); break;
    case 8: combine_kernel<8, R><<<grid, 256, 0, st>>>(y_rows, inv_row, y_shared, topk_w, residual, k, H, y_out); break;
    case 10: combine_kernel<10, R><<<grid, 256, 0, st>>>(y_rows, inv_row, y_shared, topk_w, residual, k, H, y_out); break;
    default: combine_kernel<0, R><<<grid, 256, 0, st>>>(y_rows, inv_row, y_shared, topk_w, residual, k, H, y_out);
  }
}

int moe_launch_combine(const void* y_rows, int rows_dtype, const int32_t* inv_row, const void* y_shared,
                       const float* topk_w, const float* residual, int T, int k, int H, float* y_out, hipStream_t st) {
  if (T == 0) return MOE_OK;
  if (rows_dtype == MOE_F16)
    launch_combine_t((const _Float16*)y_rows, inv_row, (const _Float16*)y_shared, topk_w, residual, T, k, H, y_out,
                     st);
  else
    launch_combine_t((const float*)y_rows, inv_row, (const float*)y_shared, topk_w, residual, T, k, H, y_out, st);
  return moe_check_launch("combine");
}

extern "C" int moe_combine(const void* y_rows, int rows_dtype, const int32_t* inv_row, const void* y_shared,
                           const float* topk_w, const float* residual, int T, int k, int H, float* y_out,
                           void* stream) {
  MOE_REQUIRE(T >= 0 && T < 65536 * 32, MOE_ESHAPE, "T=%d out of range", T);
  MOE_REQUIRE(k >= 1 && k <= MOE_MAX_K, MOE_ESHAPE, "k=%d out of [1, %d]", k, MOE_MAX_K);
  MOE_REQUIRE(H >= 4 && H % 4 == 0 && H <= MOE_MAX_H, MOE_ESHAPE, "H=%d must be a multiple of 4", H);
  MOE_REQUIRE(rows_dtype == MOE_F32 || rows_dtype == MOE_F16, MOE_EUNSUPPORTED,
              "rows_dtype=%d must be MOE_F32 or MOE_F16", rows_dtype);
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(y_rows && topk_w && y_out, MOE_EINVAL, "y_rows, topk_w and y_out are required");
  MOE_REQUIRE((inv_row == nullptr) == (y_shared == nullptr), MOE_EINVAL,
              "inv_row and y_shared are given together (prefill layout) or both NULL (decode layout)");
  MOE_REQUIRE(moe_aligned(y_rows, 16) && moe_aligned(y_out, 16) && (!residual || moe_aligned(residual, 16)) &&
                  (!y_shared || moe_aligned(y_shared, 16)),
              MOE_EALIGN, "y_rows, y_shared, residual and y_out must be 16-byte aligned");
  return moe_launch_combine(y_rows, rows_dtype, inv_row, y_shared, topk_w, residual, T, k, H, y_out,
                            moe_stream(stream));
}
