// Prefill experts: grouped GEMM over the rows that moe_permute grouped by
// expert, plus the shared expert as one more group over all T tokens.
//
// A prompt chunk of thousands of tokens routes to nearly every expert, and
// each expert's weights then serve all of the chunk's rows that chose it
// ("为什么 Strata 在小显存显卡上这么快", section "读长提示词：大块流式读取"), so
// the work is a dense contraction per expert and runs on the matrix cores.
//
// Per group g (expert g < E with rows offsets[g]..offsets[g+1], or the shared
// expert g == E with rows 0..T-1), tiles of BM = 128 rows:
//   gate/up pass: G|U = X_rows . [Wg|Wu]^T, h = fp16(silu(G) * U)  -> ws
//   down pass:    Y   = h_rows . Wd^T (fp32)                       -> y_perm / y_shared
// MFMA v_mfma_f32_32x32x16_f16.  Weights are dequantised in registers to
// fp16(s*q) (int4) or fp16(s*q+m) (int2), one rounding each; x (bf16) is
// converted to fp16 exactly when staged into LDS; accumulation is fp32.
//
// Workgroup: 4 waves, tile 128 rows x 256 weight rows; wave w owns weight
// rows nbase..nbase+63 = two 32-wide MFMA column tiles and all four 32-row
// MFMA row tiles (128 fp32 accumulators per lane).  For the gate/up pass the
// record interleaves gate and up rows in runs of 32, so a wave's two column
// tiles are gate and up of the same 32 f values and SiLU*mul happens in
// registers.  K is walked 64 at a time with the next chunk's A tile and B
// words prefetched into registers (LDS double buffer).
//
// Blocks are renumbered so that consecutive work items (the column tiles of
// one row tile, then the row tiles of one expert) land on the same XCD
// (hardware dispatch places block b on XCD b % 8): the x rows and weights a
// tile shares stay in that XCD's L2.
#include "moe_common.h"
#include "moe_sizes.h"

#define GEMM_BM MOE_GEMM_BM
#define GEMM_BN 256
#define GEMM_KC 64
#define GEMM_LDS_STRIDE 72  // halves per staged row (64 + 8 pad)

__global__ __launch_bounds__(1024) void gemm_schedule_kernel(const int32_t* __restrict__ offsets, int E, int T,
                                                             int32_t* __restrict__ tile_start) {
  __shared__ int s[2048];
  const int G = E + 1;
  for (int g = threadIdx.x; g < 2048; g += 1024) {
    int n = 0;
    if (g < E) n = (offsets[g + 1] - offsets[g] + GEMM_BM - 1) / GEMM_BM;
    else if (g == E) n = (T + GEMM_BM - 1) / GEMM_BM;
    s[g] = n;
  }
  __syncthreads();
  // inclusive scan over 2048 entries, two per thread
  for (int d = 1; d < 2048; d <<= 1) {
    const int i0 = threadIdx.x, i1 = threadIdx.x + 1024;
    const int v0 = i0 >= d ? s[i0 - d] : 0;
    const int v1 = i1 >= d ? s[i1 - d] : 0;
    __syncthreads();
    s[i0] += v0;
    s[i1] += v1;
    __syncthreads();
  }
  for (int g = threadIdx.x; g <= G; g += 1024) tile_start[g] = g == 0 ? 0 : s[g - 1];
}

template <int QFMT>
struct BRegs;  // raw weight words of one K chunk (64) for one lane and two column tiles

template <>
struct BRegs<MOE_Q4_B32> {
  uint2 q[2][2];   // [sub][block in chunk]: dwords 2hh, 2hh+1 of the block
  uint32_t s[2];   // [sub]: fp16 scales of the chunk's two blocks
};
template <>
struct BRegs<MOE_Q2_B16> {
  uint4 q[2];      // [sub]: q-unit (4 blocks)
  uint4 m[2];      // [sub]: meta-unit
};

__device__ __forceinline__ void load_b(BRegs<MOE_Q4_B32>& b, const uint8_t* rec, const MoePlanes& pl, int rows,
                                       int row0, int hh, int c, bool gu) {
  const int64_t q_off = gu ? pl.gu_q : pl.d_q, s_off = gu ? pl.gu_s : pl.d_s;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int r = row0 + 32 * sub;
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      const int kb = 2 * c + bi;
      b.q[sub][bi] = *reinterpret_cast<const uint2*>(rec + q_off + 16 * ((int64_t)kb * rows + r) + 8 * hh);
    }
    const int kb = 2 * c;
    if (gu) {  // 4-block groups: kb even -> both scales in one 4-byte word
      b.s[sub] = *reinterpret_cast<const uint32_t*>(rec + s_off + 2 * ((int64_t)(kb >> 2) * rows * 4 + 4 * r + (kb & 3)));
    } else {   // per block [kb][row]
      const uint32_t s0 = *reinterpret_cast<const uint16_t*>(rec + s_off + 2 * ((int64_t)kb * rows + r));
      const uint32_t s1 = *reinterpret_cast<const uint16_t*>(rec + s_off + 2 * ((int64_t)(kb + 1) * rows + r));
      b.s[sub] = s0 | (s1 << 16);
    }
  }
}

__device__ __forceinline__ void load_b(BRegs<MOE_Q2_B16>& b, const uint8_t* rec, const MoePlanes& pl, int rows,
                                       int row0, int hh, int c, bool gu) {
  const int64_t q_off = gu ? pl.gu_q : pl.d_q, m_off = gu ? pl.gu_s : pl.d_s;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int r = row0 + 32 * sub;
    if (gu) {  // 4-block units
      b.q[sub] = *reinterpret_cast<const uint4*>(rec + q_off + 16 * ((int64_t)c * rows + r));
      b.m[sub] = *reinterpret_cast<const uint4*>(rec + m_off + 16 * ((int64_t)c * rows + r));
    } else {   // per block [b][row]
      uint32_t qw[4], mw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qw[j] = *reinterpret_cast<const uint32_t*>(rec + q_off + 4 * ((int64_t)(4 * c + j) * rows + r));
        mw[j] = *reinterpret_cast<const uint32_t*>(rec + m_off + 4 * ((int64_t)(4 * c + j) * rows + r));
      }
      b.q[sub] = make_uint4(qw[0], qw[1], qw[2], qw[3]);
      b.m[sub] = make_uint4(mw[0], mw[1], mw[2], mw[3]);
    }
  }
  (void)hh;
}

// fp16(s*q) for 8 consecutive int4 values of one dword (natural order).
__device__ __forceinline__ half8v deq_q4(uint32_t w, half2v s2) {
  const half2v k1032 = {(_Float16)1032.f, (_Float16)1032.f};
  half8v r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    half2v q = moe_u32_as_half2(((w >> (4 * p)) & 0x000F000Fu) | MOE_F16_1024X2) - k1032;
    half2v v = q * s2;
    r[2 * p] = v[0];
    r[2 * p + 1] = v[1];
  }
  return r;
}

// fp16(s*q+m) for values 8hh..8hh+7 of one int2 block word.
__device__ __forceinline__ half8v deq_q2(uint32_t w, int hh, half2v s2, half2v m2) {
  const half2v k1024 = {(_Float16)1024.f, (_Float16)1024.f};
  const uint32_t x = w >> (8 * hh);
  half8v r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    half2v q = moe_u32_as_half2(((x >> (2 * p)) & 0x00030003u) | MOE_F16_1024X2) - k1024;
    half2v v = __builtin_elementwise_fma(q, s2, m2);
    r[2 * p] = v[0];
    r[2 * p + 1] = v[1];
  }
  return r;
}

template <int QFMT, bool GU>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const uint16_t* __restrict__ a_src, int T, int H, int F, int k,
                                                      int E, const int32_t* __restrict__ row_src,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ tile_start,
                                                      const int32_t* __restrict__ slot_table, int layer,
                                                      const uint8_t* __restrict__ pool, int64_t record_bytes,
                                                      _Float16* __restrict__ h_out, float* __restrict__ y_perm,
                                                      float* __restrict__ y_shared, int n_ntiles, int total_wg) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][GEMM_BM * GEMM_LDS_STRIDE];
  __shared__ int arow[GEMM_BM];

  // XCD-aware renumbering (total_wg is a multiple of 8)
  const int bid = blockIdx.x;
  const int work = (bid & 7) * (total_wg >> 3) + (bid >> 3);
  const int tile = work / n_ntiles, nt = work % n_ntiles;
  if (tile >= tile_start[E + 1]) return;
  int lo = 0, hi = E;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= tile) lo = mid;
    else hi = mid - 1;
  }
  const int g = lo;
  const int m0 = (tile - tile_start[g]) * GEMM_BM;
  const int Mg = g < E ? offsets[g + 1] - offsets[g] : T;
  const int mv = min(GEMM_BM, Mg - m0);
  const int gbase = g < E ? offsets[g] : T * k;  // first h row of the group

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, ln = lane & 31;
  const int K = GU ? H : F;
  const int rows = GU ? 2 * F : H;  // rows of the stored weight matrix
  const int nbase = nt * GEMM_BN + 64 * wave;
  const bool active = nbase < rows;

  if (tid < GEMM_BM) {
    int r = -1;
    if (tid < mv) {
      if (GU) r = g < E ? row_src[gbase + m0 + tid] / k : m0 + tid;
      else r = gbase + m0 + tid;
    }
    arow[tid] = r;
  }
  const int64_t slot = slot_table[(size_t)layer * (E + 1) + g];
  const uint8_t* rec = pool + slot * record_bytes;
  const MoePlanes pl = moe_planes(QFMT, H, F);
  __syncthreads();

  // A staging: thread -> (row st_r, 32 values at st_c)
  const int st_r = tid >> 1, st_c = 32 * (tid & 1);
  const int my_arow = arow[st_r];
  uint4 areg[4];
  auto load_a = [&](int c) {
    if (my_arow >= 0) {
      const uint4* p = reinterpret_cast<const uint4*>(a_src + (size_t)my_arow * K + c * GEMM_KC + st_c);
#pragma unroll
      for (int i = 0; i < 4; ++i) areg[i] = p[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) areg[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_a = [&](int stage) {
    uint4* d = reinterpret_cast<uint4*>(&As[stage][st_r * GEMM_LDS_STRIDE + st_c]);
    if constexpr (GU) {  // bf16 -> fp16
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w[4] = {areg[i].x, areg[i].y, areg[i].z, areg[i].w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          half2v h = {(_Float16)__uint_as_float(w[j] << 16), (_Float16)__uint_as_float(w[j] & 0xffff0000u)};
          o[j] = moe_half2_as_u32(h);
        }
        d[i] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = areg[i];
    }
  };

  float16v acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][s][v] = 0.f;

  const int nc = K / GEMM_KC;
  BRegs<QFMT> bcur, bnext;
  load_a(0);
  if (active) load_b(bcur, rec, pl, rows, nbase + ln, hh, 0, GU);
  store_a(0);
  __syncthreads();

  for (int c = 0; c < nc; ++c) {
    const int stage = c & 1;
    if (c + 1 < nc) {
      load_a(c + 1);
      if (active) load_b(bnext, rec, pl, rows, nbase + ln, hh, c + 1, GU);
    }
    if (active) {
      const _Float16* Ab = &As[stage][0];
      if constexpr (QFMT == MOE_Q4_B32) {
        const BRegs<MOE_Q4_B32>& B = bcur;
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            half8v bf[2];
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
              const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)(B.s[sub] >> (16 * bi)));
              const half2v s2 = {sc, sc};
              bf[sub] = deq_q4(s == 0 ? B.q[sub][bi].x : B.q[sub][bi].y, s2);
            }
            const int kk = 32 * bi + 16 * hh + 8 * s;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const half8v af = *reinterpret_cast<const half8v*>(&Ab[(32 * i + ln) * GEMM_LDS_STRIDE + kk]);
#pragma unroll
              for (int sub = 0; sub < 2; ++sub)
                acc[i][sub] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf[sub], acc[i][sub], 0, 0, 0);
            }
          }
        }
      } else {
        const BRegs<MOE_Q2_B16>& B = bcur;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          half8v bf[2];
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            const uint32_t qw = j == 0 ? B.q[sub].x : j == 1 ? B.q[sub].y : j == 2 ? B.q[sub].z : B.q[sub].w;
            const uint32_t mw = j == 0 ? B.m[sub].x : j == 1 ? B.m[sub].y : j == 2 ? B.m[sub].z : B.m[sub].w;
            const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)(mw & 0xffff));
            const _Float16 mn = __builtin_bit_cast(_Float16, (uint16_t)(mw >> 16));
            const half2v s2 = {sc, sc}, m2 = {mn, mn};
            bf[sub] = deq_q2(qw, hh, s2, m2);
          }
          const int kk = 16 * j + 8 * hh;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const half8v af = *reinterpret_cast<const half8v*>(&Ab[(32 * i + ln) * GEMM_LDS_STRIDE + kk]);
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
              acc[i][sub] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf[sub], acc[i][sub], 0, 0, 0);
          }
        }
      }
    }
    if (c + 1 < nc) store_a(stage ^ 1);
    __syncthreads();
    bcur = bnext;
  }

  if (!active) return;
  // epilogue: lane holds column ln, rows 8*(v/4) + 4*hh + v%4 of each 32-row tile
  if constexpr (GU) {
    const int f = 32 * (nbase / 64) + ln;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * i + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (r < mv) {
          const float gv = acc[i][0][v], uv = acc[i][1][v];
          h_out[(size_t)(gbase + m0 + r) * F + f] = (_Float16)(moe_silu(gv) * uv);
        }
      }
    }
  } else {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int col = nbase + 32 * sub + ln;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = 32 * i + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (r < mv) {
            if (g < E) y_perm[(size_t)(gbase + m0 + r) * H + col] = acc[i][sub][v];
            else y_shared[(size_t)(m0 + r) * H + col] = acc[i][sub][v];
          }
        }
      }
    }
  }
}

template <int QFMT>
static int launch_gemm_t(const uint16_t* x, int T, int H, int F, const int32_t* row_src, const int32_t* offsets,
                         int k, int E, const int32_t* slot_table, int layer, const void* pool, int64_t record_bytes,
                         float* y_perm, float* y_shared, void* ws, hipStream_t st) {
  int32_t* tile_start = (int32_t*)ws;
  _Float16* h = (_Float16*)((uint8_t*)ws + moe_gemm_h_offset(E));
  gemm_schedule_kernel<<<1, 1024, 0, st>>>(offsets, E, T, tile_start);
  const int max_tiles = moe_gemm_max_tiles(T, k, E);
  {
    const int nnt = (2 * F + GEMM_BN - 1) / GEMM_BN;
    const int total = (max_tiles * nnt + 7) / 8 * 8;
    gemm_kernel<QFMT, true><<<total, 256, 0, st>>>(x, T, H, F, k, E, row_src, offsets, tile_start, slot_table, layer,
                                                   (const uint8_t*)pool, record_bytes, h, y_perm, y_shared, nnt,
                                                   total);
  }
  {
    const int nnt = (H + GEMM_BN - 1) / GEMM_BN;
    const int total = (max_tiles * nnt + 7) / 8 * 8;
    gemm_kernel<QFMT, false><<<total, 256, 0, st>>>((const uint16_t*)h, T, H, F, k, E, row_src, offsets, tile_start,
                                                    slot_table, layer, (const uint8_t*)pool, record_bytes, h, y_perm,
                                                    y_shared, nnt, total);
  }
  return moe_check_launch("grouped gemm");
}

extern "C" int moe_grouped_gemm_q(const uint16_t* x, int T, int H, int F, const int32_t* row_src,
                                  const int32_t* offsets, int k, int E, const int32_t* slot_table, int layer,
                                  const void* pool, int64_t record_bytes, int qfmt, float* y_perm, float* y_shared,
                                  void* ws, size_t ws_bytes, void* stream) {
  int rc = moe_check_expert_shapes(H, F, E, k, qfmt, pool, record_bytes, slot_table, layer);
  if (rc) return rc;
  MOE_REQUIRE(T >= 0, MOE_ESHAPE, "T=%d must be >= 0", T);
  MOE_REQUIRE(((int64_t)T * k + T) * (int64_t)(H > F ? H : F) < (1ll << 31) * 8ll, MOE_ESHAPE, "T too large");
  MOE_REQUIRE((int64_t)T * k + T < (1ll << 31), MOE_ESHAPE, "T*k too large");
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(x && row_src && offsets && y_perm && y_shared, MOE_EINVAL,
              "x, row_src, offsets, y_perm and y_shared are required");
  MOE_REQUIRE(moe_aligned(x, 16), MOE_EALIGN, "x must be 16-byte aligned");
  const size_t need = moe_ws_gemm(T, k, E, F);
  MOE_REQUIRE(ws && ws_bytes >= need && moe_aligned(ws, 256), MOE_EWORKSPACE,
              "ws needs %zu bytes, 256-byte aligned", need);
  hipStream_t st = moe_stream(stream);
  if (qfmt == MOE_Q4_B32)
    return launch_gemm_t<MOE_Q4_B32>(x, T, H, F, row_src, offsets, k, E, slot_table, layer, pool, record_bytes,
                                     y_perm, y_shared, ws, st);
  return launch_gemm_t<MOE_Q2_B16>(x, T, H, F, row_src, offsets, k, E, slot_table, layer, pool, record_bytes, y_perm,
                                   y_shared, ws, st);
}
