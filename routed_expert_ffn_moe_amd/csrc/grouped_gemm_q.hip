// Prefill experts: grouped GEMM over the rows that moe_permute grouped by
// expert, plus the shared expert as one more group over all T tokens.
//
// A prompt chunk of thousands of tokens routes to nearly every expert, and
// each expert's weights then serve all of the chunk's rows that chose it
// ("为什么 Strata 在小显存显卡上这么快", section "读长提示词：大块流式读取"), so
// the work is a dense contraction per expert and runs on the matrix cores.
//
// Per group g (expert g < E with rows offsets[g]..offsets[g+1], or the shared
// expert g == E with rows 0..T-1): its ceil(M/32) row tiles of 32 are split as
// evenly as possible over ceil(M/BM) workgroup tiles:
//   gate/up pass: G|U = X_rows . [Wg|Wu]^T, h = fp16(silu(G) * U)  -> ws
//   down pass:    Y   = h_rows . Wd^T (fp32)                       -> y_perm / y_shared
// MFMA v_mfma_f32_32x32x16_f16.  Weights are dequantised in registers to
// fp16(s*q) (int4) or fp16(s*q+m) (int2), one rounding each; x (bf16) is
// converted to fp16 (exact in fp16's normal range) once, into the workspace,
// before the gate/up pass; accumulation is fp32.
//
// Two kernels compute it (gemm2_kernel is the one used; gemm_kernel, the
// first version, is kept behind MOE_GEMM_KERNEL=v1 for comparison).  Both
// use workgroups of 4 waves where wave w owns weight rows nbase..nbase+63 =
// two 32-wide MFMA column tiles over the tile's 32-row MFMA row tiles; for
// the gate/up pass the record interleaves gate and up rows in runs of 32, so
// a wave's two column tiles are gate and up of the same 32 f values and
// SiLU*mul happens in registers.  The next K chunk's A tile and B words are
// requested before the current chunk's MFMAs (A through registers into a
// double-buffered LDS tile).
//   gemm_kernel:  BM = 128 (a 160-row expert runs as 64 + 96 rows), K chunks
//                 of 128, the MFMAs of absent row tiles skipped by branches.
//   gemm2_kernel: BM = 160 (a typical expert is one tile, each dequantised
//                 weight operand feeds up to 5 MFMAs), K chunks of 64, and a
//                 K loop specialised on the row-tile count: no branches, so
//                 the compiler's waits count only the loads a step needs.
//
// Blocks are renumbered so that consecutive work items (the column tiles of
// one row tile, then the row tiles of one expert) land on the same XCD
// (hardware dispatch places block b on XCD b % 8): the x rows and weights a
// tile shares stay in that XCD's L2.
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "moe_common.h"
#include "moe_sizes.h"

#define GEMM_BM MOE_GEMM_BM
#define GEMM_BN 256
#define GEMM_KC 128
#define GEMM_NB (GEMM_KC / 32)  // int4 blocks per K chunk
#define GEMM_LDS_STRIDE 136     // halves per staged row (128 + 8 pad)

// tile_start[g] = first tile of group g (exclusive scan of ceil(M_g / BM), BM a
// multiple of 32);
// tile_info[t] = {group, first row m0, rows, first h row of the group}: the
// group's 32-row tiles split as evenly as possible over its BM-row tiles.
__global__ __launch_bounds__(1024) void gemm_schedule_kernel(const int32_t* __restrict__ offsets, int E, int T,
                                                             int k, int BM, int32_t* __restrict__ tile_start,
                                                             int4* __restrict__ tile_info) {
  __shared__ int s[2048];
  const int G = E + 1;
  for (int g = threadIdx.x; g < 2048; g += 1024) {
    int n = 0;
    if (g < E) n = (offsets[g + 1] - offsets[g] + BM - 1) / BM;
    else if (g == E) n = (T + BM - 1) / BM;
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
  for (int g = threadIdx.x; g < G; g += 1024) {
    const int t0 = g == 0 ? 0 : s[g - 1], n = s[g] - t0;
    const int Mg = g < E ? offsets[g + 1] - offsets[g] : T;
    const int gbase = g < E ? offsets[g] : T * k;
    const int nrt_g = (Mg + 31) / 32;
    for (int lt = 0; lt < n; ++lt) {
      const int rt0 = lt * nrt_g / n, nrt = (lt + 1) * nrt_g / n - rt0;
      const int m0 = 32 * rt0;
      tile_info[t0 + lt] = make_int4(g, m0, min(32 * nrt, Mg - m0), gbase);
    }
  }
}

// x (bf16) -> fp16, 8 values per thread (n8 = T * H / 8)
__global__ __launch_bounds__(256) void x_to_f16_kernel(const uint4* __restrict__ x, size_t n8, uint4* __restrict__ y) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (size_t)gridDim.x * 256) {
    const uint4 v = x[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half2v h = {(_Float16)__uint_as_float(w[j] << 16), (_Float16)__uint_as_float(w[j] & 0xffff0000u)};
      o[j] = moe_half2_as_u32(h);
    }
    y[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

template <int QFMT>
struct BRegs;  // raw weight words of one K chunk (128) for one lane and two column tiles

template <>
struct BRegs<MOE_Q4_B32> {
  uint2 q[2][GEMM_NB];   // [sub][block in chunk]: dwords 2hh, 2hh+1 of the block
  uint32_t s[2][2];      // [sub][block pair]: fp16 scales of blocks 2p, 2p+1
};
template <>
struct BRegs<MOE_Q2_B16> {
  uint4 q[2][2];         // [sub][unit]: q-unit (4 blocks)
  uint4 m[2][2];         // [sub][unit]: meta-unit
};

__device__ __forceinline__ void load_b(BRegs<MOE_Q4_B32>& b, const uint8_t* rec, const MoePlanes& pl, int rows,
                                       int row0, int hh, int c, bool gu) {
  // rec is wave-uniform and a record is < 4 GiB: 32-bit offsets
  const uint32_t q_off = (uint32_t)(gu ? pl.gu_q : pl.d_q), s_off = (uint32_t)(gu ? pl.gu_s : pl.d_s);
  const uint32_t R = (uint32_t)rows;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const uint32_t r = (uint32_t)(row0 + 32 * sub);
#pragma unroll
    for (int bi = 0; bi < GEMM_NB; ++bi) {
      const uint32_t kb = (uint32_t)(GEMM_NB * c + bi);
      b.q[sub][bi] = *reinterpret_cast<const uint2*>(rec + (q_off + 16u * (kb * R + r) + 8u * (uint32_t)hh));
    }
    const uint32_t kb = (uint32_t)(GEMM_NB * c);  // a multiple of 4
    if (gu) {  // 4-block groups: the chunk's 4 scales in one 8-byte word
      const uint2 w = *reinterpret_cast<const uint2*>(rec + (s_off + 2u * ((kb >> 2) * R * 4u + 4u * r)));
      b.s[sub][0] = w.x;
      b.s[sub][1] = w.y;
    } else {   // per block [kb][row]
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const uint32_t s0 = *reinterpret_cast<const uint16_t*>(rec + (s_off + 2u * ((kb + 2 * p) * R + r)));
        const uint32_t s1 = *reinterpret_cast<const uint16_t*>(rec + (s_off + 2u * ((kb + 2 * p + 1) * R + r)));
        b.s[sub][p] = s0 | (s1 << 16);
      }
    }
  }
}

__device__ __forceinline__ void load_b(BRegs<MOE_Q2_B16>& b, const uint8_t* rec, const MoePlanes& pl, int rows,
                                       int row0, int hh, int c, bool gu) {
  const uint32_t q_off = (uint32_t)(gu ? pl.gu_q : pl.d_q), m_off = (uint32_t)(gu ? pl.gu_s : pl.d_s);
  const uint32_t R = (uint32_t)rows;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const uint32_t r = (uint32_t)(row0 + 32 * sub);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t un = (uint32_t)(2 * c + u);  // 4-block unit (64 values of K)
      if (gu) {
        b.q[sub][u] = *reinterpret_cast<const uint4*>(rec + (q_off + 16u * (un * R + r)));
        b.m[sub][u] = *reinterpret_cast<const uint4*>(rec + (m_off + 16u * (un * R + r)));
      } else {   // per block [b][row]
        uint32_t qw[4], mw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          qw[j] = *reinterpret_cast<const uint32_t*>(rec + (q_off + 4u * ((4u * un + j) * R + r)));
          mw[j] = *reinterpret_cast<const uint32_t*>(rec + (m_off + 4u * ((4u * un + j) * R + r)));
        }
        b.q[sub][u] = make_uint4(qw[0], qw[1], qw[2], qw[3]);
        b.m[sub][u] = make_uint4(mw[0], mw[1], mw[2], mw[3]);
      }
    }
  }
  (void)hh;
}

// The nibble mask held in a register: (x & mask) | magic is then one
// v_and_or_b32 (with both operands literal constants it takes two
// instructions, the VOP3 encoding taking no literal here).
__device__ __forceinline__ uint32_t moe_vgpr_const(uint32_t c) {
  asm volatile("" : "+v"(c));
  return c;
}

// fp16(s*q) for 8 consecutive int4 values of one dword (natural order);
// m4 = 0x000F000F (in a register).
__device__ __forceinline__ half8v deq_q4(uint32_t w, half2v s2, uint32_t m4) {
  const half2v k1032 = {(_Float16)1032.f, (_Float16)1032.f};
  half8v r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    half2v q = moe_u32_as_half2(((w >> (4 * p)) & m4) | MOE_F16_1024X2) - k1032;
    half2v v = q * s2;
    r[2 * p] = v[0];
    r[2 * p + 1] = v[1];
  }
  return r;
}

// fp16(s*q+m) for values 8hh..8hh+7 of one int2 block word; m2b = 0x00030003
// (in a register).
__device__ __forceinline__ half8v deq_q2(uint32_t w, int hh, half2v s2, half2v m2, uint32_t m2b) {
  const half2v k1024 = {(_Float16)1024.f, (_Float16)1024.f};
  const uint32_t x = w >> (8 * hh);
  half8v r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    half2v q = moe_u32_as_half2(((x >> (2 * p)) & m2b) | MOE_F16_1024X2) - k1024;
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
                                                      const int4* __restrict__ tile_info,
                                                      const int32_t* __restrict__ slot_table, int layer,
                                                      const uint8_t* __restrict__ pool, int64_t record_bytes,
                                                      _Float16* __restrict__ h_out, float* __restrict__ y_perm,
                                                      float* __restrict__ y_shared, int n_ntiles, int total_wg) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][GEMM_BM * GEMM_LDS_STRIDE];
  __shared__ int arow[GEMM_BM];

  // XCD-aware renumbering: block b runs on XCD b % 8; the real work count
  // (known only here) is cut into 8 consecutive ranges, one per XCD.  The
  // grid (total_wg, a multiple of 8) is an upper bound; surplus blocks exit.
  const int bid = blockIdx.x;
  const int nwork = tile_start[E + 1] * n_ntiles;
  const int per_xcd = (nwork + 7) >> 3;
  const int idx = bid >> 3;
  const int work = (bid & 7) * per_xcd + idx;
  if (idx >= per_xcd || work >= nwork) return;
  const int tile = work / n_ntiles, nt = work % n_ntiles;
  const int4 ti = tile_info[tile];
  const int g = ti.x, m0 = ti.y, mv = ti.z, gbase = ti.w;  // gbase: first h row of the group
  const int nrt = (mv + 31) / 32;                           // row tiles present (<= 4)

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

  // A staging (fp16 rows): thread -> (row st_r, 32 values at st_c)
  const int st_r = tid >> 1, st_c = (GEMM_KC / 2) * (tid & 1);
  const int my_arow = arow[st_r];
  constexpr int NA = GEMM_KC / 16;  // uint4 (8 halves) per staging thread
  uint4 areg[NA];
  const bool st_on = st_r < 32 * nrt;  // wave-uniform: wave w stages row tile w
  auto load_a = [&](int c) {
    if (!st_on) return;
    if (my_arow >= 0) {
      const uint4* p = reinterpret_cast<const uint4*>(a_src + (size_t)my_arow * K + c * GEMM_KC + st_c);
#pragma unroll
      for (int i = 0; i < NA; ++i) areg[i] = p[i];
    } else {
#pragma unroll
      for (int i = 0; i < NA; ++i) areg[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_a = [&](int stage) {
    if (!st_on) return;
    uint4* d = reinterpret_cast<uint4*>(&As[stage][st_r * GEMM_LDS_STRIDE + st_c]);
#pragma unroll
    for (int i = 0; i < NA; ++i) d[i] = areg[i];
  };

  float16v acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][s][v] = 0.f;

  const int nc = K / GEMM_KC;
  const uint32_t m4 = moe_vgpr_const(0x000F000Fu), m2b = moe_vgpr_const(0x00030003u);
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
        for (int bi = 0; bi < GEMM_NB; ++bi) {
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            half8v bf[2];
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
              const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)(B.s[sub][bi >> 1] >> (16 * (bi & 1))));
              const half2v s2 = {sc, sc};
              bf[sub] = deq_q4(s == 0 ? B.q[sub][bi].x : B.q[sub][bi].y, s2, m4);
            }
            const int kk = 32 * bi + 16 * hh + 8 * s;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (i >= nrt) break;
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
        for (int jj = 0; jj < 8; ++jj) {
          const int u = jj >> 2, j = jj & 3;
          half8v bf[2];
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            const uint4 Q = B.q[sub][u], Mm = B.m[sub][u];
            const uint32_t qw = j == 0 ? Q.x : j == 1 ? Q.y : j == 2 ? Q.z : Q.w;
            const uint32_t mw = j == 0 ? Mm.x : j == 1 ? Mm.y : j == 2 ? Mm.z : Mm.w;
            const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)(mw & 0xffff));
            const _Float16 mn = __builtin_bit_cast(_Float16, (uint16_t)(mw >> 16));
            const half2v s2 = {sc, sc}, m2 = {mn, mn};
            bf[sub] = deq_q2(qw, hh, s2, m2, m2b);
          }
          const int kk = 16 * jj + 8 * hh;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (i >= nrt) break;
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
    _Float16* hb = h_out + (size_t)(gbase + m0) * F + f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= nrt) break;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * i + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (r < mv) {
          const float gv = acc[i][0][v], uv = acc[i][1][v];
          hb[(uint32_t)(r * F)] = (_Float16)(moe_silu_fast(gv) * uv);
        }
      }
    }
  } else {
    float* yb = g < E ? y_perm + (size_t)(gbase + m0) * H : y_shared + (size_t)m0 * H;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int col = nbase + 32 * sub + ln;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= nrt) break;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = 32 * i + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (r < mv) yb[(uint32_t)(r * H + col)] = acc[i][sub][v];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- gemm2
// The same contraction with tiles of up to 160 rows (5 MFMA row tiles) x 256
// weight rows and K chunks of 64.  Wave w owns two 32-wide column tiles (for
// gate/up: the gate and the up columns of the same 32 f values, which the
// record interleaves in runs of 32, so SiLU*mul happens in registers); each
// dequantised B operand feeds up to 5 MFMAs (a 160-row expert is one tile,
// not 64 + 96 rows) and each A operand read from LDS feeds 2.
#define G2_BM 160
#define G2_BN 256
#define G2_KC 64
#define G2_NB (G2_KC / 32)  // int4 blocks per K chunk
#define G2_STRIDE 72        // halves per staged row (64 + 8 pad)
#define G2_RT (G2_BM / 32)  // MFMA row tiles per workgroup tile
#define G2_NA ((G2_BM * G2_KC / 8 + 255) / 256)  // 16-byte A words per staging thread

template <int QFMT>
struct B2Regs;  // raw weight words of one K chunk (64) for one lane and one column tile
template <>
struct B2Regs<MOE_Q4_B32> {
  uint2 q[G2_NB];  // [block in chunk]: dwords 2hh, 2hh+1 of the block
  uint32_t s;      // fp16 scales of the chunk's two blocks
};
template <>
struct B2Regs<MOE_Q2_B16> {
  uint4 q;  // the chunk's q-unit (4 blocks of 16)
  uint4 m;  // its meta unit
};
// for a wave's two column tiles
template <int QFMT>
struct B2Pair {
  B2Regs<QFMT> t[2];
};

__device__ __forceinline__ void load_b2(B2Regs<MOE_Q4_B32>& b, const uint8_t* rec, const MoePlanes& pl, int rows,
                                        int r, int hh, int c, bool gu) {
  const uint32_t q_off = (uint32_t)(gu ? pl.gu_q : pl.d_q), s_off = (uint32_t)(gu ? pl.gu_s : pl.d_s);
  const uint32_t R = (uint32_t)rows, ur = (uint32_t)r;
#pragma unroll
  for (int bi = 0; bi < G2_NB; ++bi) {
    const uint32_t kb = (uint32_t)(G2_NB * c + bi);
    b.q[bi] = *reinterpret_cast<const uint2*>(rec + (q_off + 16u * (kb * R + ur) + 8u * (uint32_t)hh));
  }
  const uint32_t kb0 = (uint32_t)(G2_NB * c);  // even
  if (gu)  // 4-block groups [kb/4][row][4]: the two scales are half of the group's word
    b.s = *reinterpret_cast<const uint32_t*>(rec + (s_off + 2u * ((kb0 >> 2) * R * 4u + 4u * ur + (kb0 & 3u))));
  else {   // per block [kb][row]
    const uint32_t s0 = *reinterpret_cast<const uint16_t*>(rec + (s_off + 2u * (kb0 * R + ur)));
    const uint32_t s1 = *reinterpret_cast<const uint16_t*>(rec + (s_off + 2u * ((kb0 + 1u) * R + ur)));
    b.s = s0 | (s1 << 16);
  }
}

__device__ __forceinline__ void load_b2(B2Regs<MOE_Q2_B16>& b, const uint8_t* rec, const MoePlanes& pl, int rows,
                                        int r, int hh, int c, bool gu) {
  const uint32_t q_off = (uint32_t)(gu ? pl.gu_q : pl.d_q), m_off = (uint32_t)(gu ? pl.gu_s : pl.d_s);
  const uint32_t R = (uint32_t)rows, ur = (uint32_t)r, un = (uint32_t)c;  // one 4-block unit per chunk
  if (gu) {
    b.q = *reinterpret_cast<const uint4*>(rec + (q_off + 16u * (un * R + ur)));
    b.m = *reinterpret_cast<const uint4*>(rec + (m_off + 16u * (un * R + ur)));
  } else {  // per block [b][row]
    uint32_t qw[4], mw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qw[j] = *reinterpret_cast<const uint32_t*>(rec + (q_off + 4u * ((4u * un + j) * R + ur)));
      mw[j] = *reinterpret_cast<const uint32_t*>(rec + (m_off + 4u * ((4u * un + j) * R + ur)));
    }
    b.q = make_uint4(qw[0], qw[1], qw[2], qw[3]);
    b.m = make_uint4(mw[0], mw[1], mw[2], mw[3]);
  }
  (void)hh;
}

// The K loop of gemm2 for NRT row tiles: A chunks staged through registers
// into a double-buffered LDS tile (the next chunk's A and B words are
// requested before the current chunk's MFMAs), B dequantised in registers.
template <int QFMT, bool GU, int NRT>
__device__ __forceinline__ void gemm2_k_loop(const uint16_t* __restrict__ a_src, int K, int rows, const uint8_t* rec,
                                             const MoePlanes& pl, int nbase, const int* arow,
                                             _Float16 (*As)[G2_BM * G2_STRIDE], float16v (&acc)[G2_RT][2]) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int hh = lane >> 5, ln = lane & 31;
  constexpr int NW = NRT * 32 * G2_KC / 8;     // 16-byte A words of a chunk
  constexpr int NA = (NW + 255) / 256;         // per thread
  int src[NA];     // source row (clamped) of each staged word
  bool live[NA];   // the row has a source (else the word is zero)
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int i = min(tid + 256 * j, NW - 1);
    const int r = arow[i >> 3];
    live[j] = r >= 0;
    src[j] = r >= 0 ? r : 0;
  }
  uint4 areg[NA];
  auto load_a = [&](int c) {
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int i = min(tid + 256 * j, NW - 1);
      const uint4 v = *reinterpret_cast<const uint4*>(a_src + (size_t)src[j] * K + c * G2_KC + 8 * (i & 7));
      areg[j] = live[j] ? v : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_a = [&](int stage) {
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int i = tid + 256 * j;
      if (i < NW) *reinterpret_cast<uint4*>(&As[stage][(i >> 3) * G2_STRIDE + 8 * (i & 7)]) = areg[j];
    }
  };
  const int brow0 = min(nbase + ln, rows - 1), brow1 = min(nbase + 32 + ln, rows - 1);
  const int nc = K / G2_KC;
  const uint32_t m4 = moe_vgpr_const(0x000F000Fu), m2b = moe_vgpr_const(0x00030003u);
  B2Pair<QFMT> bcur, bnext;
  load_a(0);
  load_b2(bcur.t[0], rec, pl, rows, brow0, hh, 0, GU);
  load_b2(bcur.t[1], rec, pl, rows, brow1, hh, 0, GU);
  store_a(0);
  __syncthreads();
  for (int c = 0; c < nc; ++c) {
    const int stage = c & 1;
    const int cn = min(c + 1, nc - 1);  // the last chunk requests itself again (unused)
    load_a(cn);
    load_b2(bnext.t[0], rec, pl, rows, brow0, hh, cn, GU);
    load_b2(bnext.t[1], rec, pl, rows, brow1, hh, cn, GU);
    const _Float16* Ab = &As[stage][0];
    if constexpr (QFMT == MOE_Q4_B32) {
#pragma unroll
      for (int bi = 0; bi < G2_NB; ++bi) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int kk = 32 * bi + 16 * hh + 8 * s;
          half8v af[NRT];
#pragma unroll
          for (int i = 0; i < NRT; ++i) af[i] = *reinterpret_cast<const half8v*>(&Ab[(32 * i + ln) * G2_STRIDE + kk]);
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            const B2Regs<QFMT>& B = bcur.t[sub];
            const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)(B.s >> (16 * bi)));
            const half2v s2 = {sc, sc};
            const half8v bf = deq_q4(s == 0 ? B.q[bi].x : B.q[bi].y, s2, m4);
#pragma unroll
            for (int i = 0; i < NRT; ++i)
              acc[i][sub] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf, acc[i][sub], 0, 0, 0);
          }
        }
      }
    } else {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int kk = 16 * jj + 8 * hh;
        half8v af[NRT];
#pragma unroll
        for (int i = 0; i < NRT; ++i) af[i] = *reinterpret_cast<const half8v*>(&Ab[(32 * i + ln) * G2_STRIDE + kk]);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const B2Regs<QFMT>& B = bcur.t[sub];
          const uint32_t qw = jj == 0 ? B.q.x : jj == 1 ? B.q.y : jj == 2 ? B.q.z : B.q.w;
          const uint32_t mw = jj == 0 ? B.m.x : jj == 1 ? B.m.y : jj == 2 ? B.m.z : B.m.w;
          const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)(mw & 0xffff));
          const _Float16 mn = __builtin_bit_cast(_Float16, (uint16_t)(mw >> 16));
          const half2v s2 = {sc, sc}, m2 = {mn, mn};
          const half8v bf = deq_q2(qw, hh, s2, m2, m2b);
#pragma unroll
          for (int i = 0; i < NRT; ++i)
            acc[i][sub] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf, acc[i][sub], 0, 0, 0);
        }
      }
    }
    store_a(stage ^ 1);  // (after the last chunk: a harmless rewrite of the free stage)
    __syncthreads();
    bcur = bnext;
  }
}

template <int QFMT, bool GU>
__global__ __launch_bounds__(256, 2) void gemm2_kernel(const uint16_t* __restrict__ a_src, int T, int H, int F, int k,
                                                       int E, const int32_t* __restrict__ row_src,
                                                       const int32_t* __restrict__ tile_start,
                                                       const int4* __restrict__ tile_info,
                                                       const int32_t* __restrict__ slot_table, int layer,
                                                       const uint8_t* __restrict__ pool, int64_t record_bytes,
                                                       _Float16* __restrict__ h_out, float* __restrict__ y_perm,
                                                       float* __restrict__ y_shared, int n_ntiles) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][G2_BM * G2_STRIDE];
  __shared__ int arow[G2_BM];

  // XCD-aware renumbering (block b runs on XCD b % 8): the work count is cut
  // into 8 consecutive ranges, one per XCD, so that the column tiles of one
  // row tile and the row tiles of one expert share an XCD's L2
  const int bid = blockIdx.x;
  const int nwork = tile_start[E + 1] * n_ntiles;
  const int per_xcd = (nwork + 7) >> 3;
  const int idx = bid >> 3;
  const int work = (bid & 7) * per_xcd + idx;
  if (idx >= per_xcd || work >= nwork) return;
  const int tile = work / n_ntiles, nt = work % n_ntiles;
  const int4 ti = tile_info[tile];
  const int g = ti.x, m0 = ti.y, mv = ti.z, gbase = ti.w;
  const int nrt = (mv + 31) / 32;  // row tiles present (<= 5)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, ln = lane & 31;
  const int K = GU ? H : F;
  const int rows = GU ? 2 * F : H;
  const int nbase = nt * G2_BN + 64 * wave;  // this wave's 64 weight rows
  const bool active = nbase < rows;

  if (tid < G2_BM) {
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

  float16v acc[G2_RT][2];
#pragma unroll
  for (int i = 0; i < G2_RT; ++i)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][sub][v] = 0.f;
  // The K loop, specialised on the row-tile count (uniform per workgroup),
  // so that it has no branches: its loads are unconditional (indices clamped
  // into range; rows without a source are zeroed after the load) and the
  // waits the compiler places count only the loads a step really needs.
  switch (nrt) {
    case 1: gemm2_k_loop<QFMT, GU, 1>(a_src, K, rows, rec, pl, nbase, arow, As, acc); break;
    case 2: gemm2_k_loop<QFMT, GU, 2>(a_src, K, rows, rec, pl, nbase, arow, As, acc); break;
    case 3: gemm2_k_loop<QFMT, GU, 3>(a_src, K, rows, rec, pl, nbase, arow, As, acc); break;
    case 4: gemm2_k_loop<QFMT, GU, 4>(a_src, K, rows, rec, pl, nbase, arow, As, acc); break;
    default: gemm2_k_loop<QFMT, GU, 5>(a_src, K, rows, rec, pl, nbase, arow, As, acc); break;
  }

  // epilogue: lane holds column ln, rows 8*(v/4) + 4*hh + v%4 of each 32-row tile
  if (!active) return;
  if constexpr (GU) {
    const int f = 32 * (nbase / 64) + ln;
    _Float16* hb = h_out + (size_t)(gbase + m0) * F + f;
#pragma unroll
    for (int i = 0; i < G2_RT; ++i) {
      if (i >= nrt) break;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * i + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (r < mv) hb[(uint32_t)(r * F)] = (_Float16)(moe_silu_fast(acc[i][0][v]) * acc[i][1][v]);
      }
    }
  } else {
    float* yb = g < E ? y_perm + (size_t)(gbase + m0) * H : y_shared + (size_t)m0 * H;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int col = nbase + 32 * sub + ln;
#pragma unroll
      for (int i = 0; i < G2_RT; ++i) {
        if (i >= nrt) break;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = 32 * i + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (r < mv) yb[(uint32_t)(r * H + col)] = acc[i][sub][v];
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
  int4* tile_info = (int4*)((uint8_t*)ws + moe_gemm_info_offset(E));
  _Float16* h = (_Float16*)((uint8_t*)ws + moe_gemm_h_offset(T, k, E));
  uint16_t* x16 = (uint16_t*)((uint8_t*)ws + moe_gemm_x16_offset(T, k, E, F));
  const char* kv = getenv("MOE_GEMM_KERNEL");
  const bool v2 = !(kv && strcmp(kv, "v1") == 0);
  gemm_schedule_kernel<<<1, 1024, 0, st>>>(offsets, E, T, k, v2 ? G2_BM : GEMM_BM, tile_start, tile_info);
  {
    const size_t n8 = (size_t)T * H / 8;
    const int grid = (int)std::min<size_t>((n8 + 255) / 256, 4096);
    x_to_f16_kernel<<<grid, 256, 0, st>>>((const uint4*)x, n8, (uint4*)x16);
  }
  const int max_tiles = moe_gemm_max_tiles(T, k, E);  // bounds the tile count for BM >= 128
  if (v2) {
    const int nnt_gu = (2 * F + G2_BN - 1) / G2_BN, nnt_d = (H + G2_BN - 1) / G2_BN;
    const int tot_gu = (max_tiles * nnt_gu + 7) / 8 * 8, tot_d = (max_tiles * nnt_d + 7) / 8 * 8;
    gemm2_kernel<QFMT, true><<<tot_gu, 256, 0, st>>>(x16, T, H, F, k, E, row_src, tile_start, tile_info, slot_table,
                                                     layer, (const uint8_t*)pool, record_bytes, h, y_perm, y_shared,
                                                     nnt_gu);
    gemm2_kernel<QFMT, false><<<tot_d, 256, 0, st>>>((const uint16_t*)h, T, H, F, k, E, row_src, tile_start, tile_info,
                                                      slot_table, layer, (const uint8_t*)pool, record_bytes, h, y_perm,
                                                      y_shared, nnt_d);
    return moe_check_launch("grouped gemm");
  }
  {
    const int nnt = (2 * F + GEMM_BN - 1) / GEMM_BN;
    const int total = (max_tiles * nnt + 7) / 8 * 8;
    gemm_kernel<QFMT, true><<<total, 256, 0, st>>>(x16, T, H, F, k, E, row_src, offsets, tile_start, tile_info, slot_table, layer,
                                                   (const uint8_t*)pool, record_bytes, h, y_perm, y_shared, nnt,
                                                   total);
  }
  {
    const int nnt = (H + GEMM_BN - 1) / GEMM_BN;
    const int total = (max_tiles * nnt + 7) / 8 * 8;
    gemm_kernel<QFMT, false><<<total, 256, 0, st>>>((const uint16_t*)h, T, H, F, k, E, row_src, offsets, tile_start,
                                                    tile_info, slot_table, layer, (const uint8_t*)pool, record_bytes, h, y_perm,
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
  const size_t need = moe_ws_gemm(T, k, E, H, F);
  MOE_REQUIRE(ws && ws_bytes >= need && moe_aligned(ws, 256), MOE_EWORKSPACE,
              "ws needs %zu bytes, 256-byte aligned", need);
  hipStream_t st = moe_stream(stream);
  if (qfmt == MOE_Q4_B32)
    return launch_gemm_t<MOE_Q4_B32>(x, T, H, F, row_src, offsets, k, E, slot_table, layer, pool, record_bytes,
                                     y_perm, y_shared, ws, st);
  return launch_gemm_t<MOE_Q2_B16>(x, T, H, F, row_src, offsets, k, E, slot_table, layer, pool, record_bytes, y_perm,
                                   y_shared, ws, st);
}
