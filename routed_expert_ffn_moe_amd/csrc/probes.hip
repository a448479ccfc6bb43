// Measurement probes (include/moe_probes.h): the practical HBM streaming-read
// rate and the MFMA-only rate of the device, the ceilings the layer's
// kernels are compared with.  The read probe's shape (16,384 workgroups,
// eight nontemporal 16-byte loads in flight per thread) was the fastest of
// 1,024-16,384 workgroups, 4 or 8 loads, with or without the hint (6.9 TB/s
// over 4 GiB).
#include "moe_common.h"
#include "../../include/moe_probes.h"

#define PROBE_READ_BLOCKS 16384
#define PROBE_MFMA_WAVES 16  // per workgroup: 4 per SIMD

__global__ __launch_bounds__(256) void probe_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  uint32_t acc = 0u;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {  // eight 16-byte nontemporal loads in flight per thread
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = moe_ld_stream16(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ uint32_t red[4];
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(64 * PROBE_MFMA_WAVES) void probe_mfma_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  half8v a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (float)((lane + i) & 7));
    b[i] = (_Float16)(0.001f * (float)((lane * 3 + i) & 7));
  }
  float16v c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  s = moe_wave_sum(s);
  __shared__ float red[PROBE_MFMA_WAVES];
  if (lane == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < PROBE_MFMA_WAVES; ++w) t += red[w];
    sink[blockIdx.x] = t;
  }
}

static int probe_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

extern "C" int moe_probe_stream_read_blocks(void) { return PROBE_READ_BLOCKS; }

extern "C" int moe_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  MOE_REQUIRE(src && sink, MOE_EINVAL, "src and sink are required");
  MOE_REQUIRE(moe_aligned(src, 16) && bytes % 16 == 0, MOE_EALIGN, "src 16-byte aligned, bytes a multiple of 16");
  probe_read_kernel<<<PROBE_READ_BLOCKS, 256, 0, moe_stream(stream)>>>((const uint4*)src, bytes / 16, sink);
  return moe_check_launch("probe stream read");
}

extern "C" int moe_probe_mfma_blocks(void) { return probe_cus(); }

extern "C" double moe_probe_mfma_flops(int iters) {
  return (double)probe_cus() * PROBE_MFMA_WAVES * (double)iters * 4.0 * 32768.0;
}

extern "C" int moe_probe_mfma(int iters, float* sink, void* stream) {
  MOE_REQUIRE(sink, MOE_EINVAL, "sink is required");
  MOE_REQUIRE(iters >= 1, MOE_EINVAL, "iters must be >= 1");
  probe_mfma_kernel<<<probe_cus(), 64 * PROBE_MFMA_WAVES, 0, moe_stream(stream)>>>(iters, sink);
  return moe_check_launch("probe mfma");
}
