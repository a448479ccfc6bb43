// The pre-norm of a stack of layers: xn[t] = x[t] / sqrt(mean_h(x[t]^2) + eps)
// (unit gain), in fp32 or rounded once to bf16 (round to nearest even) for a
// prefill chunk's router and grouped GEMM.  The pages do not describe the
// non-MoE parts of a layer; without a norm a chain of SwiGLU layers, which
// are quadratic in x, overflows within a few layers.
#include "moe_common.h"
#include "moe_kernels.h"

// one workgroup of 256 threads per token, fixed-order fp32 reduction
template <bool BF16>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, int H, float eps,
                                                      void* __restrict__ out) {
  __shared__ float part[4];
  const float* xr = x + (size_t)blockIdx.x * H;
  float s = 0.f;
  for (int h = threadIdx.x; h < H; h += 256) s = fmaf(xr[h], xr[h], s);
  s = moe_wave_sum(s);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  const float ms = ((part[0] + part[1]) + (part[2] + part[3])) / (float)H;
  const float inv = 1.0f / sqrtf(ms + eps);
  for (int h = threadIdx.x; h < H; h += 256) {
    const float v = xr[h] * inv;
    if (BF16) {  // round to nearest even (finite v)
      const uint32_t u = __float_as_uint(v);
      ((uint16_t*)out)[(size_t)blockIdx.x * H + h] = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    } else {
      ((float*)out)[(size_t)blockIdx.x * H + h] = v;
    }
  }
}

int moe_launch_rmsnorm(const float* x, int T, int H, float eps, void* out, int out_dtype, hipStream_t st) {
  if (T == 0) return MOE_OK;
  if (out_dtype == MOE_BF16)
    rmsnorm_kernel<true><<<T, 256, 0, st>>>(x, H, eps, out);
  else
    rmsnorm_kernel<false><<<T, 256, 0, st>>>(x, H, eps, out);
  return moe_check_launch("rmsnorm");
}

extern "C" int moe_rmsnorm(const float* x, int T, int H, float eps, void* out, int out_dtype, void* stream) {
  MOE_REQUIRE(T >= 0, MOE_ESHAPE, "T=%d must be >= 0", T);
  MOE_REQUIRE(H >= 1 && H <= MOE_MAX_H, MOE_ESHAPE, "H=%d out of [1, %d]", H, MOE_MAX_H);
  MOE_REQUIRE(out_dtype == MOE_F32 || out_dtype == MOE_BF16, MOE_EUNSUPPORTED, "unknown out_dtype %d", out_dtype);
  MOE_REQUIRE(eps >= 0.f, MOE_EINVAL, "eps must be >= 0");
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(x && out, MOE_EINVAL, "x and out are required");
  MOE_REQUIRE((const void*)x != out, MOE_EINVAL, "out may not alias x");
  return moe_launch_rmsnorm(x, T, H, eps, out, out_dtype, moe_stream(stream));
}
