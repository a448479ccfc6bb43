// Shared device and host helpers of libmoe (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/moe.h"

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

#define MOE_WAVE 64

// ---------------------------------------------------------------- host side

// Records an error message for moe_last_error() and returns `code`.
int moe_fail(int code, const char* fmt, ...);
// Returns MOE_OK, or MOE_EHIP with the runtime's message after a launch.
int moe_check_launch(const char* what);

#define MOE_REQUIRE(cond, code, ...)                 \
  do {                                               \
    if (!(cond)) return moe_fail((code), __VA_ARGS__); \
  } while (0)

static inline hipStream_t moe_stream(void* s) { return (hipStream_t)s; }
static inline bool moe_aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
static inline size_t moe_align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Shape checks shared by the expert entry points.
int moe_check_expert_shapes(int H, int F, int E, int k, int qfmt, const void* pool,
                            int64_t record_bytes, const int32_t* slot_table, int layer);

// ---------------------------------------------------------------- device side

__device__ __forceinline__ float moe_bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ half2v moe_u32_as_half2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
__device__ __forceinline__ uint32_t moe_half2_as_u32(half2v h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ float moe_f16_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// fp32 dot of two fp16 pairs plus an fp32 addend (v_dot2_f32_f16).
__device__ __forceinline__ float moe_dot2(half2v a, half2v b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}

__device__ __forceinline__ float moe_silu(float z) { return z / (1.0f + expf(-z)); }
// SiLU with the hardware exp and reciprocal (about 1 ulp in fp32), for values
// that are rounded to fp16 right after; z -> -inf gives -0, z -> +inf gives z.
__device__ __forceinline__ float moe_silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Order-preserving map of a (non-NaN) fp32 to uint32; -0 and +0 map alike.
__device__ __forceinline__ uint32_t moe_f32_order_key(float f) {
  uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float moe_order_key_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t moe_shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, m, MOE_WAVE);
  hi = __shfl_xor(hi, m, MOE_WAVE);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t moe_wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = moe_shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float moe_wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, MOE_WAVE);
  return v;
}

// ---------------------------------------------------------------- record layout
// Byte offsets of the planes of one record (include/moe.h).
struct MoePlanes {
  int64_t gu_q, d_q, gu_s, d_s;
};
__host__ __device__ __forceinline__ MoePlanes moe_planes(int qfmt, int H, int F) {
  int64_t HF = (int64_t)H * F;
  MoePlanes p;
  if (qfmt == MOE_Q4_B32) {
    p.gu_q = 0; p.d_q = HF; p.gu_s = 3 * HF / 2; p.d_s = 3 * HF / 2 + HF / 8;
  } else {
    p.gu_q = 0; p.d_q = HF / 2; p.gu_s = 3 * HF / 4; p.d_s = 5 * HF / 4;
  }
  return p;
}

// int4 nibble pairs: word w holds values v0..v7 of a block as
// v0:[0,4) v2:[4,8) v4:[8,12) v6:[12,16) v1:[16,20) v3:[20,24) v5:[24,28) v7:[28,32).
// (w >> 4p) & 0x000F000F puts (v_{2p}, v_{2p+1}) in the low / high half-words.
// OR-ing 0x6400 into a half makes the fp16 value 1024 + nibble.
#define MOE_F16_1024X2 0x64006400u

// Loads of data that is read once (expert weights in decode, router rows):
// the nontemporal hint lets the caches evict these lines first.  A probe
// streaming 4 GiB measured 6.9 TB/s with the hint against 6.2 TB/s without.
typedef uint32_t moe_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 moe_ld_stream16(const void* p) {
  const moe_u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const moe_u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint32_t moe_ld_stream4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ uint32_t moe_ld_stream2(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
}

// 8 consecutive activations as fp32 (16-byte aligned source).
__device__ __forceinline__ void moe_load8(const float* p, float v[8]) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void moe_load8(const uint16_t* p, float v[8]) {
  uint4 a = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
