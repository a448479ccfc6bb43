// Decode / verify experts: gather-GEMV over the distinct experts that 1..8
// tokens chose, plus the shared expert.
//
// A decode step reads each chosen expert once and is bound by memory traffic:
// a token touches 480 routed experts over 48 layers ("为什么 Strata 在小显存显
// 卡上这么快", section "问题：1250 亿参数，12 GB 显存"), and in a verify step
// only the extra tokens' experts add reads (same page, section "先猜，再检查").
//
// Inner loop.  Lane l of a wave owns weight row r and walks the K blocks of
// that row; the 16-byte block (kb, r) is one coalesced 128-bit load per lane
// because the record stores blocks in [kb][row] order.  Nibbles become fp16
// 1024+n by OR-ing the fp16 exponent of 1024 into them; the activation side
// is prepared once per token in fp16 pairs ordered like the nibble pairs (odd
// pairs of each word pre-divided by 16 so that a mask without shift serves
// them), and the constant that the 1024 (and the +8 offset) contribute is
// removed with one per-block correction:
//   int4: blk = sum dot2(1024+n|1024+16n, x~) - c,  acc += s * blk
//   int2: blk = sum dot2(1024+c*q, x~) - c0,       acc += s * blk + m * sum(x^)
// Sums are fp32; x and the SwiGLU intermediate are rounded once to fp16.
#include "moe_common.h"
#include "moe_sizes.h"
#include "moe_kernels.h"

#define GEMV_WAVES 4

struct GemvPlan {
  int* base;
  int umax;
  __device__ __forceinline__ int& U() const { return base[0]; }
  __device__ __forceinline__ int& expert(int u) const { return base[1 + u]; }
  __device__ __forceinline__ int& ntok(int u) const { return base[1 + umax + u]; }
  __device__ __forceinline__ int& tok(int u, int i) const { return base[1 + 2 * umax + u * MOE_MAX_DECODE_T + i]; }
  __device__ __forceinline__ int& jpos(int u, int i) const {
    return base[1 + 2 * umax + umax * MOE_MAX_DECODE_T + u * MOE_MAX_DECODE_T + i];
  }
};

// ---------------------------------------------------------------- activation prep
// Prepares block `blk` of a K-vector whose values b[0..31] (int4) or
// b[0..15] (int2) are given: the fp16 pairs go to pairs[] and the block's
// correction to corr[blk].  A prepared vector is K fp16 followed by one
// float2 per block.
template <int QFMT>
__device__ void moe_prep_block(const float* b, int blk, uint32_t* pairs, float2* corr) {
  if (QFMT == MOE_Q4_B32) {
    uint32_t* p = pairs + 16 * blk;
    const half2v k0 = {(_Float16)1032.f, (_Float16)1032.f};
    const half2v k1 = {(_Float16)1152.f, (_Float16)1152.f};
    float c = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half2v a0 = {(_Float16)b[8 * j + 0], (_Float16)b[8 * j + 1]};
      half2v a1 = {(_Float16)(b[8 * j + 2] * 0.0625f), (_Float16)(b[8 * j + 3] * 0.0625f)};
      half2v a2 = {(_Float16)b[8 * j + 4], (_Float16)b[8 * j + 5]};
      half2v a3 = {(_Float16)(b[8 * j + 6] * 0.0625f), (_Float16)(b[8 * j + 7] * 0.0625f)};
      p[4 * j + 0] = moe_half2_as_u32(a0);
      p[4 * j + 1] = moe_half2_as_u32(a1);
      p[4 * j + 2] = moe_half2_as_u32(a2);
      p[4 * j + 3] = moe_half2_as_u32(a3);
      c = moe_dot2(a0, k0, c);
      c = moe_dot2(a1, k1, c);
      c = moe_dot2(a2, k0, c);
      c = moe_dot2(a3, k1, c);
    }
    corr[blk] = make_float2(c, 0.f);
  } else {
    uint32_t* p = pairs + 8 * blk;
    const half2v k1024 = {(_Float16)1024.f, (_Float16)1024.f};
    float c0 = 0.f, sx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float mul = (i & 3) == 0 ? 1.f : (i & 3) == 1 ? 0.25f : (i & 3) == 2 ? 0.0625f : 0.015625f;
      const float cc = 1.f / mul;
      half2v a = {(_Float16)(b[2 * i] * mul), (_Float16)(b[2 * i + 1] * mul)};
      p[i] = moe_half2_as_u32(a);
      const half2v kc = {(_Float16)cc, (_Float16)cc};
      c0 = moe_dot2(a, k1024, c0);
      sx = moe_dot2(a, kc, sx);
    }
    corr[blk] = make_float2(c0, sx);
  }
}

// block 0: plan of distinct experts; block 1+t: prepared x of token t.
template <int QFMT>
__global__ __launch_bounds__(256) void gemv_prep_kernel(const float* __restrict__ x, int T, int H,
                                                        const int32_t* __restrict__ topk_idx, int k, int E,
                                                        int* __restrict__ plan_base, int umax,
                                                        uint8_t* __restrict__ xprep, size_t xprep_stride) {
  if (blockIdx.x == 0) {
    __shared__ int ent[MOE_MAX_DECODE_T * MOE_MAX_K];
    __shared__ int first[MOE_MAX_DECODE_T * MOE_MAX_K];
    __shared__ int rank[MOE_MAX_DECODE_T * MOE_MAX_K];
    GemvPlan P{plan_base, umax};
    const int n = T * k;
    const int i = threadIdx.x;
    if (i < n) ent[i] = topk_idx[i];
    __syncthreads();
    if (i < n) {
      int f = 1;
      for (int j = 0; j < i; ++j) f &= (ent[j] != ent[i]);
      first[i] = f;
    }
    __syncthreads();
    if (i < n && first[i]) {
      int r = 0;
      for (int j = 0; j < n; ++j) r += (first[j] && ent[j] < ent[i]);
      rank[i] = r;
    }
    __syncthreads();
    if (i < n && first[i]) {
      const int u = rank[i];
      const int e = ent[i];
      P.expert(u) = e;
      int c = 0;
      for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j)
          if (ent[t * k + j] == e && c < MOE_MAX_DECODE_T) {
            P.tok(u, c) = t;
            P.jpos(u, c) = j;
            ++c;
          }
      P.ntok(u) = c;
    }
    if (i == 0) {
      int U = 0;
      for (int j = 0; j < n; ++j) U += first[j];
      P.U() = U + 1;
      P.expert(U) = E;  // the shared expert
      P.ntok(U) = T;
      for (int t = 0; t < T; ++t) {
        P.tok(U, t) = t;
        P.jpos(U, t) = k;
      }
    }
    return;
  }
  const int t = blockIdx.x - 1;
  uint8_t* out = xprep + (size_t)t * xprep_stride;
  const int nblk = H / (QFMT == MOE_Q4_B32 ? 32 : 16);
  const int bsz = QFMT == MOE_Q4_B32 ? 32 : 16;
  for (int b = threadIdx.x; b < nblk; b += 256)
    moe_prep_block<QFMT>(x + (size_t)t * H + (size_t)b * bsz, b, (uint32_t*)out, (float2*)(out + 2 * (size_t)H));
}

// ---------------------------------------------------------------- inner products
// One block of 32 (int4) / one q-unit of 64 (int2) for NT token vectors.
template <int MAXT>
__device__ __forceinline__ void moe_q4_block(uint4 q, float s, const uint8_t* const* prep, int kb, int H,
                                             int ntok, float* acc) {
  const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
  half2v wp[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = qw[j], w8 = qw[j] >> 8;
    wp[4 * j + 0] = moe_u32_as_half2((w & 0x000F000Fu) | MOE_F16_1024X2);
    wp[4 * j + 1] = moe_u32_as_half2((w & 0x00F000F0u) | MOE_F16_1024X2);
    wp[4 * j + 2] = moe_u32_as_half2((w8 & 0x000F000Fu) | MOE_F16_1024X2);
    wp[4 * j + 3] = moe_u32_as_half2((w8 & 0x00F000F0u) | MOE_F16_1024X2);
  }
#pragma unroll
  for (int i = 0; i < MAXT; ++i) {
    if (i < ntok) {
      const uint4* xp = reinterpret_cast<const uint4*>(prep[i] + 64 * (size_t)kb);
      const float c = reinterpret_cast<const float2*>(prep[i] + 2 * (size_t)H)[kb].x;
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 xv = xp[j];
        d = moe_dot2(wp[4 * j + 0], moe_u32_as_half2(xv.x), d);
        d = moe_dot2(wp[4 * j + 1], moe_u32_as_half2(xv.y), d);
        d = moe_dot2(wp[4 * j + 2], moe_u32_as_half2(xv.z), d);
        d = moe_dot2(wp[4 * j + 3], moe_u32_as_half2(xv.w), d);
      }
      acc[i] = fmaf(s, d - c, acc[i]);
    }
  }
}

template <int MAXT>
__device__ __forceinline__ void moe_q2_unit(uint4 q, uint4 meta, const uint8_t* const* prep, int u4, int K,
                                            int ntok, float* acc) {
  const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
  const uint32_t mw[4] = {meta.x, meta.y, meta.z, meta.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // block 4*u4 + j
    const uint32_t w = qw[j], w8 = qw[j] >> 8;
    half2v wp[8];
    wp[0] = moe_u32_as_half2((w & 0x00030003u) | MOE_F16_1024X2);
    wp[1] = moe_u32_as_half2((w & 0x000C000Cu) | MOE_F16_1024X2);
    wp[2] = moe_u32_as_half2((w & 0x00300030u) | MOE_F16_1024X2);
    wp[3] = moe_u32_as_half2((w & 0x00C000C0u) | MOE_F16_1024X2);
    wp[4] = moe_u32_as_half2((w8 & 0x00030003u) | MOE_F16_1024X2);
    wp[5] = moe_u32_as_half2((w8 & 0x000C000Cu) | MOE_F16_1024X2);
    wp[6] = moe_u32_as_half2((w8 & 0x00300030u) | MOE_F16_1024X2);
    wp[7] = moe_u32_as_half2((w8 & 0x00C000C0u) | MOE_F16_1024X2);
    const float s = moe_f16_to_f32((uint16_t)(mw[j] & 0xffff));
    const float m = moe_f16_to_f32((uint16_t)(mw[j] >> 16));
    const int blk = 4 * u4 + j;
#pragma unroll
    for (int i = 0; i < MAXT; ++i) {
      if (i < ntok) {
        const uint4* xp = reinterpret_cast<const uint4*>(prep[i] + 32 * (size_t)blk);
        const float2 c = reinterpret_cast<const float2*>(prep[i] + 2 * (size_t)K)[blk];
        const uint4 x0 = xp[0], x1 = xp[1];
        float d = 0.f;
        d = moe_dot2(wp[0], moe_u32_as_half2(x0.x), d);
        d = moe_dot2(wp[1], moe_u32_as_half2(x0.y), d);
        d = moe_dot2(wp[2], moe_u32_as_half2(x0.z), d);
        d = moe_dot2(wp[3], moe_u32_as_half2(x0.w), d);
        d = moe_dot2(wp[4], moe_u32_as_half2(x1.x), d);
        d = moe_dot2(wp[5], moe_u32_as_half2(x1.y), d);
        d = moe_dot2(wp[6], moe_u32_as_half2(x1.z), d);
        d = moe_dot2(wp[7], moe_u32_as_half2(x1.w), d);
        acc[i] = fmaf(s, d - c.x, fmaf(m, c.y, acc[i]));
      }
    }
  }
}

// Row r of a [kb][row]-stored matrix with `rows` rows and K columns, dotted
// with the prepared vectors, over this wave's share of K.  Returns partials
// in acc[i].
// `grouped`: the gate/up planes keep scales in 4-block groups [kb/4][row][4]
// and int2 words / (s, m) in 4-block units; the down planes store them per
// block [kb][row].
template <int QFMT, int MAXT>
__device__ __forceinline__ void moe_row_dot(const uint8_t* __restrict__ rec, int64_t q_off, int64_t s_off,
                                            int rows, int K, int r, int wave, const uint8_t* const* prep,
                                            int ntok, float* acc, bool grouped) {
  if (QFMT == MOE_Q4_B32) {
    const int KB = K / 32;
    const int per = KB / GEMV_WAVES;  // K % 128 == 0 -> KB % 4 == 0
    const int kb0 = wave * per;
    for (int g = kb0; g < kb0 + per; g += 4) {  // kb0 and per are multiples of 4? per may not be
      const int n = min(4, kb0 + per - g);
      uint4 qv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (u < n) qv[u] = *reinterpret_cast<const uint4*>(rec + q_off + 16 * ((int64_t)(g + u) * rows + r));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (u < n) {
          const int kb = g + u;
          const int64_t si = grouped ? (int64_t)(kb >> 2) * rows * 4 + 4 * r + (kb & 3) : (int64_t)kb * rows + r;
          const uint16_t sb = *reinterpret_cast<const uint16_t*>(rec + s_off + 2 * si);
          moe_q4_block<MAXT>(qv[u], moe_f16_to_f32(sb), prep, kb, K, ntok, acc);
        }
      }
    }
  } else {
    const int U4 = K / 64;
    const int per = (U4 + GEMV_WAVES - 1) / GEMV_WAVES;
    const int u0 = wave * per, u1 = min(U4, u0 + per);
    for (int u = u0; u < u1; ++u) {
      uint4 q, m;
      if (grouped) {
        q = *reinterpret_cast<const uint4*>(rec + q_off + 16 * ((int64_t)u * rows + r));
        m = *reinterpret_cast<const uint4*>(rec + s_off + 16 * ((int64_t)u * rows + r));
      } else {
        uint32_t qw[4], mw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          qw[j] = *reinterpret_cast<const uint32_t*>(rec + q_off + 4 * ((int64_t)(4 * u + j) * rows + r));
          mw[j] = *reinterpret_cast<const uint32_t*>(rec + s_off + 4 * ((int64_t)(4 * u + j) * rows + r));
        }
        q = make_uint4(qw[0], qw[1], qw[2], qw[3]);
        m = make_uint4(mw[0], mw[1], mw[2], mw[3]);
      }
      moe_q2_unit<MAXT>(q, m, prep, u, K, ntok, acc);
    }
  }
}

// ---------------------------------------------------------------- gate/up
// Workgroup (u, rg): distinct expert u, GU rows 64rg .. 64rg+63, i.e. gate and
// up rows of f = 32rg .. 32rg+31.  Wave w takes a quarter of K.  The result
// h = silu(g) * u is written prepared for the down projection (it is exactly
// down-K block rg for int4, blocks 2rg and 2rg+1 for int2).
template <int QFMT>
__global__ __launch_bounds__(256) void gemv_gu_kernel(int H, int F, int E, const int32_t* __restrict__ slot_table,
                                                      int layer, const uint8_t* __restrict__ pool,
                                                      int64_t record_bytes, int* __restrict__ plan_base, int umax,
                                                      const uint8_t* __restrict__ xprep, size_t xprep_stride,
                                                      uint8_t* __restrict__ hprep, size_t hprep_stride) {
  __shared__ float red[GEMV_WAVES][MOE_MAX_DECODE_T][64];
  __shared__ float hs[MOE_MAX_DECODE_T][32];
  GemvPlan P{plan_base, umax};
  const int u = blockIdx.x, rg = blockIdx.y;
  if (u >= P.U()) return;
  const int e = P.expert(u);
  const int ntok = P.ntok(u);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t slot = slot_table[(size_t)layer * (E + 1) + e];
  const uint8_t* rec = pool + slot * record_bytes;
  const MoePlanes pl = moe_planes(QFMT, H, F);
  const uint8_t* prep[MOE_MAX_DECODE_T];
#pragma unroll
  for (int i = 0; i < MOE_MAX_DECODE_T; ++i) prep[i] = xprep + (size_t)P.tok(u, i < ntok ? i : 0) * xprep_stride;
  float acc[MOE_MAX_DECODE_T];
#pragma unroll
  for (int i = 0; i < MOE_MAX_DECODE_T; ++i) acc[i] = 0.f;
  const int r = 64 * rg + lane;
  moe_row_dot<QFMT, MOE_MAX_DECODE_T>(rec, pl.gu_q, pl.gu_s, 2 * F, H, r, wave, prep, ntok, acc, true);
#pragma unroll
  for (int i = 0; i < MOE_MAX_DECODE_T; ++i) red[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave == 0) {
    for (int i = 0; i < ntok; ++i) {
      const float v = red[0][i][lane] + red[1][i][lane] + red[2][i][lane] + red[3][i][lane];
      const float up = __shfl(v, (lane + 32) & 63, 64);
      if (lane < 32) hs[i][lane] = moe_silu(v) * up;
    }
  }
  __syncthreads();
  // prepare h blocks for the down projection
  const int nb = QFMT == MOE_Q4_B32 ? 1 : 2;
  for (int job = threadIdx.x; job < ntok * nb; job += 256) {
    const int i = job / nb, b = job % nb;
    uint8_t* out = hprep + ((size_t)u * MOE_MAX_DECODE_T + i) * hprep_stride;
    const int blk = QFMT == MOE_Q4_B32 ? rg : 2 * rg + b;
    moe_prep_block<QFMT>(&hs[i][16 * b], blk, (uint32_t*)out, (float2*)(out + 2 * (size_t)F));
  }
}

// ---------------------------------------------------------------- down
// Workgroup (u, rg): output rows 64rg .. 64rg+63 of expert u for its tokens.
template <int QFMT>
__global__ __launch_bounds__(256) void gemv_down_kernel(int H, int F, int E, int k,
                                                        const int32_t* __restrict__ slot_table, int layer,
                                                        const uint8_t* __restrict__ pool, int64_t record_bytes,
                                                        int* __restrict__ plan_base, int umax,
                                                        const uint8_t* __restrict__ hprep, size_t hprep_stride,
                                                        float* __restrict__ y_parts) {
  __shared__ float red[GEMV_WAVES][MOE_MAX_DECODE_T][64];
  GemvPlan P{plan_base, umax};
  const int u = blockIdx.x, rg = blockIdx.y;
  if (u >= P.U()) return;
  const int e = P.expert(u);
  const int ntok = P.ntok(u);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t slot = slot_table[(size_t)layer * (E + 1) + e];
  const uint8_t* rec = pool + slot * record_bytes;
  const MoePlanes pl = moe_planes(QFMT, H, F);
  const uint8_t* prep[MOE_MAX_DECODE_T];
#pragma unroll
  for (int i = 0; i < MOE_MAX_DECODE_T; ++i) prep[i] = hprep + ((size_t)u * MOE_MAX_DECODE_T + i) * hprep_stride;
  float acc[MOE_MAX_DECODE_T];
#pragma unroll
  for (int i = 0; i < MOE_MAX_DECODE_T; ++i) acc[i] = 0.f;
  const int r = 64 * rg + lane;
  moe_row_dot<QFMT, MOE_MAX_DECODE_T>(rec, pl.d_q, pl.d_s, H, F, r, wave, prep, ntok, acc, false);
#pragma unroll
  for (int i = 0; i < MOE_MAX_DECODE_T; ++i) red[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave == 0) {
    for (int i = 0; i < ntok; ++i) {
      const float v = red[0][i][lane] + red[1][i][lane] + red[2][i][lane] + red[3][i][lane];
      const int t = P.tok(u, i), j = P.jpos(u, i);
      y_parts[((size_t)t * (k + 1) + j) * H + r] = v;
    }
  }
}

// ---------------------------------------------------------------- launcher
template <int QFMT>
static int launch_gemv_t(const float* x, int T, int H, int F, const int32_t* topk_idx, int k, int E,
                         const int32_t* slot_table, int layer, const void* pool, int64_t record_bytes,
                         float* y_parts, void* ws, hipStream_t st) {
  const MoeGemvLayout L = moe_gemv_layout(T, k, H, F, QFMT);
  uint8_t* w = (uint8_t*)ws;
  int* plan = (int*)(w + L.plan);
  gemv_prep_kernel<QFMT><<<T + 1, 256, 0, st>>>(x, T, H, topk_idx, k, E, plan, L.umax, w + L.xprep, L.xprep_stride);
  gemv_gu_kernel<QFMT><<<dim3(L.umax, 2 * F / 64), 256, 0, st>>>(
      H, F, E, slot_table, layer, (const uint8_t*)pool, record_bytes, plan, L.umax, w + L.xprep, L.xprep_stride,
      w + L.hprep, L.hprep_stride);
  gemv_down_kernel<QFMT><<<dim3(L.umax, H / 64), 256, 0, st>>>(H, F, E, k, slot_table, layer, (const uint8_t*)pool,
                                                               record_bytes, plan, L.umax, w + L.hprep,
                                                               L.hprep_stride, y_parts);
  return moe_check_launch("expert gemv");
}

int moe_launch_gemv(const float* x, int T, int H, int F, const int32_t* topk_idx, int k, int E,
                    const int32_t* slot_table, int layer, const void* pool, int64_t record_bytes, int qfmt,
                    float* y_parts, void* ws, hipStream_t st) {
  if (qfmt == MOE_Q4_B32)
    return launch_gemv_t<MOE_Q4_B32>(x, T, H, F, topk_idx, k, E, slot_table, layer, pool, record_bytes, y_parts, ws, st);
  return launch_gemv_t<MOE_Q2_B16>(x, T, H, F, topk_idx, k, E, slot_table, layer, pool, record_bytes, y_parts, ws, st);
}

extern "C" int moe_expert_gemv_q(const float* x, int T, int H, int F, const int32_t* topk_idx, int k, int E,
                                 const int32_t* slot_table, int layer, const void* pool, int64_t record_bytes,
                                 int qfmt, float* y_parts, void* ws, size_t ws_bytes, void* stream) {
  int rc = moe_check_expert_shapes(H, F, E, k, qfmt, pool, record_bytes, slot_table, layer);
  if (rc) return rc;
  MOE_REQUIRE(T >= 1 && T <= MOE_MAX_DECODE_T, MOE_ESHAPE, "T=%d out of [1, %d]", T, MOE_MAX_DECODE_T);
  MOE_REQUIRE(x && topk_idx && y_parts, MOE_EINVAL, "x, topk_idx and y_parts are required");
  MOE_REQUIRE(moe_aligned(x, 16) && moe_aligned(y_parts, 4), MOE_EALIGN, "x must be 16-byte aligned");
  const size_t need = moe_ws_gemv(T, k, H, F, qfmt);
  MOE_REQUIRE(ws && ws_bytes >= need && moe_aligned(ws, 256), MOE_EWORKSPACE,
              "ws needs %zu bytes, 256-byte aligned", need);
  return moe_launch_gemv(x, T, H, F, topk_idx, k, E, slot_table, layer, pool, record_bytes, qfmt, y_parts, ws,
                         moe_stream(stream));
}
