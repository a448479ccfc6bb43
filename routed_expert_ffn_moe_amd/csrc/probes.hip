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

// ---------------------------------------------------------------- exchange
// The all-to-all hand-offs of the persistent decode kernel with no other work:
// one 512-thread workgroup per CU (G of them, all resident), tagged 8-byte
// words (tag = round + 1 in the high half), relaxed agent-scope stores and
// loads, each thread polling its own words until they carry the round's tag
// (or a later one),
// then one workgroup barrier per round.  Patterns: 0 = x (every workgroup
// publishes 2,048 / G words to each of the 8 per-XCD copies and reads the
// 2,048 words of its XCD's copy), 1 = logits (512 words, likewise), 2 =
// partial sums (every workgroup writes 2,048 words and reads its 2,048 / G
// rows of all G producers).  ticks[g]: the 100 MHz wall-clock ticks
// workgroup g spent on the rounds; err[0] counts workgroups whose wait ran
// past its bound (the probe then stops).
#define PROBE_XCHG_SPIN (1 << 18)
__global__ __launch_bounds__(512) void probe_exchange_kernel(int pattern, int rounds, unsigned long long* buf,
                                                             long long* ticks, int* err) {
  const int g = blockIdx.x, G = gridDim.x, tid = threadIdx.x;
  const int xcc = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 7;
  const int NW = pattern == 1 ? 512 : 2048;  // words of the exchanged vector
  const int per = NW / G;                    // words each workgroup publishes (or rows it reads, pattern 2)
  const long long t0 = __builtin_amdgcn_s_memrealtime();
  for (int r = 0; r < rounds; ++r) {
    const unsigned long long tag = (unsigned long long)(r + 1) << 32;
    if (pattern < 2) {
      for (int i = tid; i < 8 * per; i += 512) {  // my words, into all 8 copies
        const int c = i / per, w = g * per + i % per;
        __hip_atomic_store(buf + (size_t)c * NW + w, tag | (unsigned)(g + w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      for (int i = tid; i < 2048; i += 512)
        __hip_atomic_store(buf + (size_t)g * 2048 + i, tag | (unsigned)i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    bool ok = true;
    // my words to poll: pattern < 2: the NW words of my XCD's copy; pattern
    // 2: rows g * per .. of every producer (G * per = 2,048 words)
    for (int i0 = 0; i0 < (pattern < 2 ? NW : 2048); i0 += 4 * 512) {
      unsigned long long w[4];
      bool need[4];
      size_t off[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = i0 + tid + 512 * q;
        need[q] = i < (pattern < 2 ? NW : 2048);
        const int ic = need[q] ? i : 0;
        off[q] = pattern < 2 ? (size_t)xcc * NW + ic : (size_t)(ic / per) * 2048 + (size_t)g * per + ic % per;
      }
      for (int it = 0;; ++it) {
        bool any = false;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (need[q]) w[q] = __hip_atomic_load(buf + off[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          // (a word may already carry a later round's tag: rounds here are not
          // chained by data, so a fast producer can run one round ahead)
          need[q] = need[q] && (w[q] >> 32) < (unsigned long long)(r + 1);
          any |= need[q];
        }
        if (!any) break;
        if (it > PROBE_XCHG_SPIN) { ok = false; break; }
      }
    }
    if (!__syncthreads_and(ok)) {
      if (tid == 0) atomicAdd(err, 1);
      break;
    }
  }
  if (tid == 0) ticks[g] = __builtin_amdgcn_s_memrealtime() - t0;
}

__global__ void probe_exchange_clear_kernel(unsigned long long* buf, size_t n, int* err) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) buf[i] = 0ull;
  if (blockIdx.x == 0 && threadIdx.x == 0) *err = 0;
}

extern "C" int moe_probe_exchange_blocks(void) { return probe_cus(); }
extern "C" size_t moe_probe_exchange_ws_bytes(void) {
  const size_t G = (size_t)probe_cus();
  return (G * 2048 > 8 * 2048 ? G * 2048 : 8 * 2048) * 8;
}

extern "C" int moe_probe_exchange(int pattern, int rounds, void* ws, size_t ws_bytes, long long* ticks, int* err,
                                  void* stream) {
  MOE_REQUIRE(pattern >= 0 && pattern <= 2, MOE_EINVAL, "pattern %d must be 0, 1 or 2", pattern);
  MOE_REQUIRE(rounds >= 1, MOE_EINVAL, "rounds must be >= 1");
  MOE_REQUIRE(ws && ticks && err, MOE_EINVAL, "ws, ticks and err are required");
  MOE_REQUIRE(ws_bytes >= moe_probe_exchange_ws_bytes() && moe_aligned(ws, 8), MOE_EWORKSPACE,
              "ws needs %zu bytes, 8-byte aligned", moe_probe_exchange_ws_bytes());
  const int G = probe_cus();
  MOE_REQUIRE(G <= 512 && 2048 % G == 0 && 512 % G == 0, MOE_EUNSUPPORTED,
              "the exchange probe needs a CU count dividing 512 (have %d)", G);
  int per_cu = 0;
  MOE_REQUIRE(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)probe_exchange_kernel, 512, 0) ==
                      hipSuccess && per_cu >= 1,
              MOE_EUNSUPPORTED, "the exchange probe's workgroups cannot all be resident");
  hipStream_t st = moe_stream(stream);
  probe_exchange_clear_kernel<<<256, 256, 0, st>>>((unsigned long long*)ws, ws_bytes / 8, err);
  probe_exchange_kernel<<<G, 512, 0, st>>>(pattern, rounds, (unsigned long long*)ws, ticks, err);
  return moe_check_launch("probe exchange");
}
