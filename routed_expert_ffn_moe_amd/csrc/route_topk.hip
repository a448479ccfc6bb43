// Router logits, top-k selection and softmax weights.
//
// The router picks 10 of 512 experts per token in every layer ("Strata开源运行
// 时：12GB显卡跑动125B参数Qwen3模型", section "模型本身：稀疏MoE带来的计算与存
// 储鸿沟"; "为什么 Strata 在小显存显卡上这么快", section "问题：1250 亿参数，
// 12 GB 显存").  Selection is on the fp32 logits, larger first, ties to the
// lower expert index; the weights are the softmax of the chosen logits.
#include "moe_common.h"
#include "moe_sizes.h"
#include "moe_kernels.h"

// ---------------------------------------------------------------- logits, few tokens
// One wave per router row e (4 rows per 256-thread workgroup).  Lane l owns the
// 8 columns 512c + 8l .. +8 of every 512-column chunk c (the last chunk may be
// partial), accumulates them sequentially for each token and the wave sums the
// 64 lane partials.
template <typename XT, int MAXT>
__global__ __launch_bounds__(256) void router_gemv_kernel(const XT* __restrict__ x, int T, int H,
                                                          const uint16_t* __restrict__ wr,
                                                          const float* __restrict__ bias, int E,
                                                          float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  float acc[MAXT];
#pragma unroll
  for (int t = 0; t < MAXT; ++t) acc[t] = 0.f;
  const uint16_t* row = wr + (size_t)e * H;
  for (int h0 = 8 * lane; h0 < H; h0 += 512) {  // H % 8 == 0: h0 < H implies h0 + 8 <= H
    uint4 wv = *reinterpret_cast<const uint4*>(row + h0);
    float w[8];
    uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[2 * i] = __uint_as_float(ww[i] << 16);
      w[2 * i + 1] = __uint_as_float(ww[i] & 0xffff0000u);
    }
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      if (t < T) {
        const XT* xr = x + (size_t)t * H + h0;
        float xv[8];
        moe_load8(xr, xv);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[t] = fmaf(xv[i], w[i], acc[t]);
      }
    }
  }
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    if (t < T) {
      float s = moe_wave_sum(acc[t]);
      if (lane == 0) logits[(size_t)t * E + e] = s + b;
    }
  }
}

// ---------------------------------------------------------------- logits, many tokens
// ---------------------------------------------------------------- logits, bf16 chunks
// x (bf16) . Wr^T (bf16) on the matrix cores (v_mfma_f32_32x32x16_bf16): the
// bf16 x bf16 products are exact and accumulate in fp32, like the VALU path
// (only the summation order differs).  Workgroup tile 128 tokens x 128
// experts, wave (wm, wn) owns tokens 64wm.. and experts 64wn.. (2 x 2 MFMA
// tiles).  Both operands go straight from global memory into registers: an
// MFMA sums over K, so A and B only have to agree on the K order, and within
// each 32 of K lane group hh = lane / 32 holds K values 16hh + 8s + i in step
// s (i < 8) -- 32 contiguous bytes of its row.  K is walked 64 at a time with
// the next chunk prefetched.  Rows past T and experts past E are clamped on
// load and not stored.  Needs H % 64 == 0.
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
__global__ __launch_bounds__(256, 2) void router_mfma_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                             const uint16_t* __restrict__ wr,
                                                             const float* __restrict__ bias, int E,
                                                             float* __restrict__ logits) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1, ln = lane & 31, hh = lane >> 5;
  const int t0 = blockIdx.x * 128 + 64 * wm, e0 = blockIdx.y * 128 + 64 * wn;
  const uint16_t* ap[2];
  const uint16_t* bp[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    ap[i] = x + (size_t)min(t0 + 32 * i + ln, T - 1) * H + 16 * hh;
    bp[i] = wr + (size_t)min(e0 + 32 * i + ln, E - 1) * H + 16 * hh;
  }
  float16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  // chunk of 64: 2 sub-chunks of 32, 2 uint4 (steps) each
  uint4 a[2][4], b[2][4], an[2][4], bn[2][4];
  auto load = [&](uint4 (&A)[2][4], uint4 (&B)[2][4], int c) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4* pa = reinterpret_cast<const uint4*>(ap[i] + c * 64 + 32 * q);
        const uint4* pb = reinterpret_cast<const uint4*>(bp[i] + c * 64 + 32 * q);
        A[i][2 * q] = pa[0];
        A[i][2 * q + 1] = pa[1];
        B[i][2 * q] = pb[0];
        B[i][2 * q + 1] = pb[1];
      }
  };
  const int nc = H / 64;  // even: H is a multiple of 128
  auto mfmas = [&](const uint4 (&A)[2][4], const uint4 (&B)[2][4]) {
#pragma unroll
    for (int s8 = 0; s8 < 4; ++s8)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8v, A[i][s8]),
                                                             __builtin_bit_cast(bf16x8v, B[j][s8]), acc[i][j], 0, 0, 0);
  };
  // two register buffers in turn (no copy between them, which would make
  // the compiler wait for the prefetch at the end of every chunk); every
  // prefetch is unconditional (the last chunks request themselves again)
  // and issued before the MFMAs of the chunk in hand
  load(a, b, 0);
  for (int c = 0; c < nc; c += 2) {
    load(an, bn, min(c + 1, nc - 1));
    __builtin_amdgcn_sched_barrier(0);
    mfmas(a, b);
    load(a, b, min(c + 2, nc - 1));
    __builtin_amdgcn_sched_barrier(0);
    mfmas(an, bn);
  }
  // lane holds expert column ln, tokens 8*(v/4) + 4*hh + v%4 of each 32 x 32 tile
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = e0 + 32 * j + ln;
    if (e >= E) continue;
    const float be = bias ? bias[e] : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = t0 + 32 * i + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (t < T) logits[(size_t)t * E + e] = acc[i][j][v] + be;
      }
  }
}

// 64 tokens x 64 experts per workgroup, K staged through LDS 32 at a time;
// each thread owns 4 tokens x 4 experts.
template <typename XT>
__global__ __launch_bounds__(256) void router_tiled_kernel(const XT* __restrict__ x, int T, int H,
                                                           const uint16_t* __restrict__ wr,
                                                           const float* __restrict__ bias, int E,
                                                           float* __restrict__ logits) {
  __shared__ float xs[64][33];
  __shared__ float ws[64][33];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < H; k0 += 32) {
    // each thread stages 8 x values and 8 router values
    {
      const int r = tid >> 2, c = (tid & 3) * 8;
      float v[8];
      if (t0 + r < T) moe_load8(x + (size_t)(t0 + r) * H + k0 + c, v);
      else for (int i = 0; i < 8; ++i) v[i] = 0.f;
      for (int i = 0; i < 8; ++i) xs[r][c + i] = v[i];
      float w[8];
      if (e0 + r < E) moe_load8(wr + (size_t)(e0 + r) * H + k0 + c, w);
      else for (int i = 0; i < 8; ++i) w[i] = 0.f;
      for (int i = 0; i < 8; ++i) ws[r][c + i] = w[i];
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[ty * 4 + i][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ws[tx * 4 + j][kk];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) logits[(size_t)t * E + e] = acc[i][j] + (bias ? bias[e] : 0.f);
    }
  }
}

// ---------------------------------------------------------------- top-k
// One wave per token.  Lane l holds the keys of experts l, l+64, ...; a key is
// (order-preserving logit bits) << 32 | ~e, so the wave maximum is the larger
// logit and, among equal logits, the lower index.  k rounds of wave argmax.
__device__ void moe_topk_wave(const float* __restrict__ lg, int E, int k, int32_t* __restrict__ idx_out,
                              float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  uint64_t key[MOE_MAX_E / 64];
#pragma unroll
  for (int i = 0; i < MOE_MAX_E / 64; ++i) {
    const int e = lane + 64 * i;
    key[i] = (e < E) ? (((uint64_t)moe_f32_order_key(lg[e]) << 32) | (uint32_t)(~(uint32_t)e)) : 0ull;
  }
  float chosen[MOE_MAX_K];
  int chosen_e[MOE_MAX_K];
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    if (j < k) {
      uint64_t m = 0;
#pragma unroll
      for (int i = 0; i < MOE_MAX_E / 64; ++i) m = key[i] > m ? key[i] : m;
      m = moe_wave_max_u64(m);
      const uint32_t e = ~(uint32_t)m;
      chosen_e[j] = (int)e;
      chosen[j] = moe_order_key_f32((uint32_t)(m >> 32));
#pragma unroll
      for (int i = 0; i < MOE_MAX_E / 64; ++i)
        if (key[i] == m) key[i] = 0ull;
    }
  }
  if (lane == 0) {
    float z[MOE_MAX_K];
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
      if (j < k) {
        z[j] = expf(chosen[j] - chosen[0]);
        sum += z[j];
      }
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
      if (j < k) {
        idx_out[j] = chosen_e[j];
        w_out[j] = z[j] / sum;
      }
    }
  }
}

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   int32_t* __restrict__ idx, float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  moe_topk_wave(logits + (size_t)t * E, E, k, idx + (size_t)t * k, w + (size_t)t * k);
}

// ---------------------------------------------------------------- launcher
int moe_launch_route(const void* x, int x_dtype, int T, int H, const uint16_t* w_router, const float* bias,
                     int E, int k, int32_t* topk_idx, float* topk_w, float* logits, hipStream_t st) {
  if (T <= MOE_MAX_DECODE_T) {
    dim3 grid((E + 3) / 4);
    if (x_dtype == MOE_F32)
      router_gemv_kernel<float, MOE_MAX_DECODE_T><<<grid, 256, 0, st>>>((const float*)x, T, H, w_router, bias, E, logits);
    else
      router_gemv_kernel<uint16_t, MOE_MAX_DECODE_T><<<grid, 256, 0, st>>>((const uint16_t*)x, T, H, w_router, bias, E, logits);
  } else if (x_dtype == MOE_BF16 && H % 64 == 0) {
    dim3 grid((T + 127) / 128, (E + 127) / 128);
    router_mfma_kernel<<<grid, 256, 0, st>>>((const uint16_t*)x, T, H, w_router, bias, E, logits);
  } else {
    dim3 grid((T + 63) / 64, (E + 63) / 64);
    if (x_dtype == MOE_F32)
      router_tiled_kernel<float><<<grid, 256, 0, st>>>((const float*)x, T, H, w_router, bias, E, logits);
    else
      router_tiled_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)x, T, H, w_router, bias, E, logits);
  }
  int rc = moe_check_launch("router logits");
  if (rc) return rc;
  topk_kernel<<<(T + 3) / 4, 256, 0, st>>>(logits, T, E, k, topk_idx, topk_w);
  return moe_check_launch("top-k");
}

extern "C" int moe_route_topk(const void* x, int x_dtype, int T, int H, const uint16_t* w_router,
                              const float* bias, int E, int k, int32_t* topk_idx, float* topk_w,
                              float* logits_out, void* ws, size_t ws_bytes, void* stream) {
  MOE_REQUIRE(x_dtype == MOE_F32 || x_dtype == MOE_BF16, MOE_EUNSUPPORTED, "x_dtype %d", x_dtype);
  MOE_REQUIRE(T >= 0, MOE_ESHAPE, "T=%d must be >= 0", T);
  MOE_REQUIRE(H >= 128 && H <= MOE_MAX_H && H % 128 == 0, MOE_ESHAPE, "H=%d must be a multiple of 128 in [128, %d]", H, MOE_MAX_H);
  MOE_REQUIRE(E >= 1 && E <= MOE_MAX_E, MOE_ESHAPE, "E=%d out of [1, %d]", E, MOE_MAX_E);
  MOE_REQUIRE(k >= 1 && k <= MOE_MAX_K && k <= E, MOE_ESHAPE, "k=%d out of [1, min(E, %d)]", k, MOE_MAX_K);
  MOE_REQUIRE((int64_t)T * E < (1ll << 31), MOE_ESHAPE, "T*E too large");
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(x && w_router && topk_idx && topk_w, MOE_EINVAL, "x, w_router, topk_idx and topk_w are required");
  MOE_REQUIRE(moe_aligned(x, 16) && moe_aligned(w_router, 16), MOE_EALIGN, "x and w_router must be 16-byte aligned");
  float* logits = logits_out;
  if (!logits) {
    MOE_REQUIRE(ws && ws_bytes >= moe_ws_route(T, E), MOE_EWORKSPACE, "ws needs %zu bytes", moe_ws_route(T, E));
    logits = (float*)ws;
  }
  return moe_launch_route(x, x_dtype, T, H, w_router, bias, E, k, topk_idx, topk_w, logits, moe_stream(stream));
}
