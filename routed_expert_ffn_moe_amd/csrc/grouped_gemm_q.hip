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
//   down pass:    Y   = h_rows . Wd^T (fp32 sums, stored fp32 or fp16) -> y_perm / y_shared
// MFMA v_mfma_f32_32x32x16_f16.  Weights are dequantised in registers to
// fp16(s*q) (int4) or fp16(s*q+m) (int2), one rounding each; x (bf16) is
// converted to fp16 (exact in fp16's normal range) once, into the workspace,
// before the gate/up pass; accumulation is fp32.
//
// gemm3_kernel uses workgroups of 4 waves where wave w owns weight rows
// nbase..nbase+63 = two 32-wide MFMA column tiles over the tile's 32-row MFMA
// row tiles; for the gate/up pass the record interleaves gate and up rows in
// runs of 32, so a wave's two column tiles are gate and up of the same 32 f
// values and SiLU*mul happens in registers.  Tiles hold up to BM = 192 rows
// (an expert of a chunk that routes about 160 rows to each expert is one
// tile, and each dequantised weight operand feeds up to 6 MFMAs), K chunks of
// 64.  A chunks are copied from global memory straight into two LDS stages,
// one chunk ahead of the MFMAs (the weight words likewise into two register
// sets), and the K loop is specialised on the row-tile count, with no
// branches.
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

// tile_start[g] = first tile of group g (exclusive scan of ceil(M_g / BM), BM a
// multiple of 32);
// tile_info[t] = {group, first row m0, rows, first h row of the group}: the
// group's 32-row tiles split as evenly as possible over its BM-row tiles.
__device__ __forceinline__ void gemm_schedule(const int32_t* __restrict__ offsets, int E, int T, int k, int BM,
                                              int32_t* __restrict__ tile_start, int4* __restrict__ tile_info) {
  // thread t owns groups 2t and 2t + 1 (E + 1 <= 2048 groups); one scan:
  // within the wave (shuffles), then over the 16 waves' totals
  __shared__ int wsum[16];
  const int G = E + 1;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int n[2], Mg[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int g = 2 * t + j;
    Mg[j] = g < E ? offsets[g + 1] - offsets[g] : g == E ? T : 0;
    n[j] = (Mg[j] + BM - 1) / BM;
  }
  const int v = n[0] + n[1];
  int x = v;  // inclusive scan over the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  int start = before + x - v;  // first tile of group 2t
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int g = 2 * t + j;
    if (g <= G) tile_start[g] = start;  // tile_start[G] = the tile count (n = 0 there)
    if (g < G) {
      const int gbase = g < E ? offsets[g] : T * k;
      const int nrt_g = (Mg[j] + 31) / 32;
      for (int lt = 0; lt < n[j]; ++lt) {
        const int rt0 = lt * nrt_g / n[j], nrt = (lt + 1) * nrt_g / n[j] - rt0;
        const int m0 = 32 * rt0;
        tile_info[start + lt] = make_int4(g, m0, min(32 * nrt, Mg[j] - m0), gbase);
      }
    }
    start += n[j];
  }
}

// Before the two passes, one launch: workgroup 0 builds the tile schedule
// while the others convert x (bf16) to fp16, 8 values per thread
// (n8 = T * H / 8), grid-stride.
__global__ __launch_bounds__(1024) void gemm_prepare_kernel(const int32_t* __restrict__ offsets, int E, int T, int k,
                                                            int BM, int32_t* __restrict__ tile_start,
                                                            int4* __restrict__ tile_info, const uint4* __restrict__ x,
                                                            size_t n8, uint4* __restrict__ y) {
  if (blockIdx.x == 0) {
    gemm_schedule(offsets, E, T, k, BM, tile_start, tile_info);
    return;
  }
  const size_t stride = (size_t)(gridDim.x - 1) * 1024;
  for (size_t i = (size_t)(blockIdx.x - 1) * 1024 + threadIdx.x; i < n8; i += stride) {
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

// ---------------------------------------------------------------- tile kernel
// Tiles of up to 192 rows (6 MFMA row tiles; 160 for int2) x 256 weight rows,
// K chunks of 64.  Wave w owns two 32-wide column tiles (for gate/up: the gate
// and the up columns of the same 32 f values, which the record interleaves in
// runs of 32, so SiLU*mul happens in registers); each dequantised B operand
// feeds up to 6 MFMAs and each A operand read from LDS feeds 2.  An expert of
// up to 192 rows is one tile, so its weights are read and dequantised once.
typedef _Float16 g3_f16x4 __attribute__((ext_vector_type(4)));
typedef float g3_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t g3_u32x4 __attribute__((ext_vector_type(4)));
#define G3_BM 192  // rows of a staged A chunk (the largest tile)
#define G3_BN 256
#define G3_KC 64
#define G3_NB (G3_KC / 32)              // int4 blocks per K chunk
// MFMA row tiles per workgroup tile: 6 for int4; 5 for int2, whose raw
// weight words of a K chunk take more registers (two 16-byte words per
// column tile)
template <int QFMT>
constexpr int g3_rt() { return QFMT == MOE_Q4_B32 ? 6 : 5; }
#define G3_STAGE_B (G3_BM * G3_KC * 2)  // bytes of one staged A chunk
#define G3_EPI_WAVE_B (32 * 128)        // a wave's output staging in the down epilogue
static_assert(4 * G3_EPI_WAVE_B <= G3_STAGE_B, "the down epilogue stages in one A stage");

template <int QFMT>
struct B2Regs;  // raw weight words of one K chunk (64) for one lane and one column tile
template <>
struct B2Regs<MOE_Q4_B32> {
  uint2 q[G3_NB];  // [block in chunk]: dwords 2hh, 2hh+1 of the block
  uint32_t s;      // fp16 scales of the chunk's two blocks (down: the first block's)
  uint32_t s1;     // down: the second block's scale, kept apart so that the two
                   // loads are not combined (and waited for) as they are issued
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
  for (int bi = 0; bi < G3_NB; ++bi) {
    const uint32_t kb = (uint32_t)(G3_NB * c + bi);
    b.q[bi] = *reinterpret_cast<const uint2*>(rec + (q_off + 16u * (kb * R + ur) + 8u * (uint32_t)hh));
  }
  const uint32_t kb0 = (uint32_t)(G3_NB * c);  // even
  if (gu)  // 4-block groups [kb/4][row][4]: the two scales are half of the group's word
    b.s = *reinterpret_cast<const uint32_t*>(rec + (s_off + 2u * ((kb0 >> 2) * R * 4u + 4u * ur + (kb0 & 3u))));
  else {   // per block [kb][row]
    b.s = *reinterpret_cast<const uint16_t*>(rec + (s_off + 2u * (kb0 * R + ur)));
    b.s1 = *reinterpret_cast<const uint16_t*>(rec + (s_off + 2u * ((kb0 + 1u) * R + ur)));
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

// s_waitcnt on the vector-memory count alone (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt and lgkmcnt at their maxima, so not waited on).
template <int N>
__device__ __forceinline__ void g3_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

#define G3_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// The K loop for NRT row tiles.  A chunks go straight from global memory into
// two LDS stages (global_load_lds, 16 bytes per lane, through no registers);
// the B words (raw quantised words, dequantised in registers) into two
// register sets; both one chunk ahead of the MFMAs.  Staged layout: row r of a
// chunk (64 halves = eight 16-byte units) at r * 128 bytes, its logical unit u
// at physical unit u ^ ((r >> 1) & 7), so that the 16 rows one ds_read_b128
// phase touches fall on 16 distinct 4-bank groups.  One load instruction of a
// wave fills 64 consecutive units (8 rows).
// Step c: wait for this wave's loads of chunk c, barrier (every wave's chunk
// c has landed, and every wave is done with the stage chunk c + 1
// overwrites), request B and then A of chunk c + 1, then the MFMAs of chunk
// c.  Requests past the last chunk repeat the last one.
template <int QFMT, bool GU, int NRT, int RT>
__device__ __forceinline__ void gemm3_k_loop(const uint8_t* a_bytes, int K, int rows, const uint8_t* rec,
                                             const MoePlanes& pl, int nbase, const int* arow, uint8_t* As0,
                                             uint8_t* As1, float16v (&acc)[RT][2]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, ln = lane & 31;
  // this lane's source for each of its NRT staging loads: tile row
  // 32j + 8*wave + lane/8, logical unit (lane & 7) ^ (that row's swizzle);
  // rows without a source read row 0 (their results are never stored)
  uint32_t voff[NRT];
  {
    const uint32_t u = (uint32_t)((lane & 7) ^ ((4 * wave + (lane >> 4)) & 7));
#pragma unroll
    for (int j = 0; j < NRT; ++j) {
      const int r = arow[32 * j + 8 * wave + (lane >> 3)];
      voff[j] = (uint32_t)(r < 0 ? 0 : r) * (uint32_t)(2 * K) + 16u * u;
    }
  }
  // byte offsets in a stage of this lane's A fragments (row tile 0) for the
  // four MFMA k-steps of a chunk
  uint32_t aoff[4];
  {
    const int sw = (ln >> 1) & 7;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int u = QFMT == MOE_Q4_B32 ? 4 * (q >> 1) + 2 * hh + (q & 1) : 2 * q + hh;
      aoff[q] = (uint32_t)(ln * 128 + 16 * (u ^ sw));
    }
  }
  const int brow0 = min(nbase + ln, rows - 1), brow1 = min(nbase + 32 + ln, rows - 1);
  const int nc = K / G3_KC;
  const uint32_t m4 = moe_vgpr_const(0x000F000Fu), m2b = moe_vgpr_const(0x00030003u);
  B2Pair<QFMT> b0, b1;

  auto issue_a = [&](int c, uint8_t* stage) {
    const uint8_t* src = a_bytes + (size_t)c * (G3_KC * 2);
    uint8_t* dst = stage + 1024 * wave;
#pragma unroll
    for (int j = 0; j < NRT; ++j) __builtin_amdgcn_global_load_lds(src + voff[j], G3_LDS(dst + 4096 * j), 16, 0, 0);
  };
  auto issue_b = [&](int c, B2Pair<QFMT>& b) {
    load_b2(b.t[0], rec, pl, rows, brow0, hh, c, GU);
    load_b2(b.t[1], rec, pl, rows, brow1, hh, c, GU);
  };
  auto compute = [&](const uint8_t* Ab, const B2Pair<QFMT>& b) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      half8v bf[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const B2Regs<QFMT>& B = b.t[sub];
        if constexpr (QFMT == MOE_Q4_B32) {
          const int bi = q >> 1, s = q & 1;
          const _Float16 sc = __builtin_bit_cast(
              _Float16, (uint16_t)(GU ? B.s >> (16 * bi) : bi == 0 ? B.s : B.s1));
          const half2v s2 = {sc, sc};
          bf[sub] = deq_q4(s == 0 ? B.q[bi].x : B.q[bi].y, s2, m4);
        } else {
          const uint32_t qw = q == 0 ? B.q.x : q == 1 ? B.q.y : q == 2 ? B.q.z : B.q.w;
          const uint32_t mw = q == 0 ? B.m.x : q == 1 ? B.m.y : q == 2 ? B.m.z : B.m.w;
          const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)(mw & 0xffff));
          const _Float16 mn = __builtin_bit_cast(_Float16, (uint16_t)(mw >> 16));
          const half2v s2 = {sc, sc}, m2 = {mn, mn};
          bf[sub] = deq_q2(qw, hh, s2, m2, m2b);
        }
      }
#pragma unroll
      for (int i = 0; i < NRT; ++i) {
        const half8v af = *reinterpret_cast<const half8v*>(Ab + aoff[q] + 4096 * i);
        // weights as the first operand: the accumulators come out transposed
        // (a lane holds one token row and 16 weight rows), so that the
        // epilogue stores 4 consecutive output columns per instruction
        acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[0], af, acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[1], af, acc[i][1], 0, 0, 0);
      }
    }
  };
  // one step: chunk c from stage `cur` with B words `bcur`, after requesting
  // B of chunk c + 1 into `bnext` and A of chunk c + 1 into stage `nxt`.  The
  // two stages are separate LDS arrays, alternating at compile time, so that
  // the compiler can tell the stage being read from the one being filled and
  // does not wait for the fill before reading.
  auto step = [&](int c, const uint8_t* cur, uint8_t* nxt, const B2Pair<QFMT>& bcur, B2Pair<QFMT>& bnext) {
    g3_wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    const int cn = min(c + 1, nc - 1);
    issue_b(cn, bnext);
    issue_a(cn, nxt);
    // keep the requests ahead of the MFMAs (the scheduler would sink them)
    __builtin_amdgcn_sched_barrier(0);
    compute(cur, bcur);
  };
  issue_b(0, b0);
  issue_a(0, As0);
  int c = 0;
  for (; c + 2 <= nc; c += 2) {
    step(c, As0, As1, b0, b1);
    step(c + 1, As1, As0, b1, b0);
  }
  if (c < nc) step(c, As0, As1, b0, b1);
  // no staging load may still be writing LDS when the workgroup ends
  g3_wait_vmcnt<0>();
}

// y_f16: the down pass writes its output rows as fp16 (else fp32).
template <int QFMT, bool GU>
__global__ __launch_bounds__(256, 2) void gemm3_kernel(const uint16_t* __restrict__ a_src, int T, int H, int F, int k,
                                                       int E, const int32_t* __restrict__ row_src,
                                                       const int32_t* __restrict__ tile_start,
                                                       const int4* __restrict__ tile_info,
                                                       const int32_t* __restrict__ slot_table, int layer,
                                                       const uint8_t* __restrict__ pool, int64_t record_bytes,
                                                       _Float16* __restrict__ h_out, void* __restrict__ y_perm,
                                                       void* __restrict__ y_shared, int y_f16, int n_ntiles) {
  __shared__ __attribute__((aligned(1024))) uint8_t As0[G3_STAGE_B];
  __shared__ __attribute__((aligned(1024))) uint8_t As1[G3_STAGE_B];
  __shared__ int arow[G3_BM];

  // XCD-aware renumbering (block b runs on XCD b % 8): the work count is cut
  // into 8 consecutive ranges, one per XCD, so that the column tiles of one
  // row tile and the row tiles of one expert share an XCD's L2
  const int bid = blockIdx.x;
  const int nwork = tile_start[E + 1] * n_ntiles;
  const int per_xcd = (nwork + 7) >> 3;
  const int idx = bid >> 3;
  const int work = (bid & 7) * per_xcd + idx;
  if (idx >= per_xcd || work >= nwork) return;
  // tiles in reverse order: the shared expert's (all full) run first, so
  // that the last, partly filled round of workgroups holds lighter tiles
  const int tile = tile_start[E + 1] - 1 - work / n_ntiles, nt = work % n_ntiles;
  const int4 ti = tile_info[tile];
  const int g = ti.x, m0 = ti.y, mv = ti.z, gbase = ti.w;
  const int nrt = (mv + 31) / 32;  // row tiles present (<= g3_rt<QFMT>())

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, ln = lane & 31;
  const int K = GU ? H : F;
  const int rows = GU ? 2 * F : H;
  const int nbase = nt * G3_BN + 64 * wave;  // this wave's 64 weight rows
  const bool active = nbase < rows;

  if (tid < G3_BM) {
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

  constexpr int RT = g3_rt<QFMT>();
  float16v acc[RT][2];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][sub][v] = 0.f;
  // the K loop, specialised on the row-tile count (uniform per workgroup)
  const uint8_t* ab = reinterpret_cast<const uint8_t*>(a_src);
  switch (nrt) {
    case 1: gemm3_k_loop<QFMT, GU, 1, RT>(ab, K, rows, rec, pl, nbase, arow, As0, As1, acc); break;
    case 2: gemm3_k_loop<QFMT, GU, 2, RT>(ab, K, rows, rec, pl, nbase, arow, As0, As1, acc); break;
    case 3: gemm3_k_loop<QFMT, GU, 3, RT>(ab, K, rows, rec, pl, nbase, arow, As0, As1, acc); break;
    case 4: gemm3_k_loop<QFMT, GU, 4, RT>(ab, K, rows, rec, pl, nbase, arow, As0, As1, acc); break;
    case 5: gemm3_k_loop<QFMT, GU, 5, RT>(ab, K, rows, rec, pl, nbase, arow, As0, As1, acc); break;
    default:
      if constexpr (RT >= 6) gemm3_k_loop<QFMT, GU, 6, RT>(ab, K, rows, rec, pl, nbase, arow, As0, As1, acc);
      break;
  }

  // epilogue: lane (ln, hh) holds token row 32*i + ln of row tile i and, in
  // acc[i][sub][4*c + e], weight row nbase + 32*sub + 8*c + 4*hh + e: four
  // consecutive output columns per c
  if constexpr (GU) {
    if (!active) return;
    // gate rows in sub 0, the matching up rows in sub 1 (interleaved per 32)
    _Float16* hb = h_out + (size_t)(gbase + m0) * F + 32 * (nbase / 64) + 4 * hh;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      if (i >= nrt) break;
      const int r = 32 * i + ln;
      if (r >= mv) continue;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        g3_f16x4 hv;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hv[e] = (_Float16)(moe_silu_fast(acc[i][0][4 * c + e]) * acc[i][1][4 * c + e]);
        *reinterpret_cast<g3_f16x4*>(hb + (uint32_t)(r * F + 8 * c)) = hv;
      }
    }
  } else {
    // Each wave stages 32 rows x 128 bytes of its output (one row tile in
    // fp16, half of one in fp32) in LDS, 16-byte unit u of row r at unit
    // u ^ (r & 7) (no bank conflicts for the 8- and 16-byte writes of 8
    // consecutive rows, nor for the reads), and writes them back 16 bytes
    // per lane: one store instruction covers whole 128-byte segments of 8
    // rows (straight from the accumulators it would cover 16 bytes in each
    // of 32 rows).  The LDS accesses stay inside the wave, which executes
    // them in order.  Written once, read once by the combine, far larger
    // than the caches: nontemporal, so that they do not displace weights.
    __syncthreads();  // every wave is done reading the last A stage
    if (!active) return;
    const size_t ybase = (g < E ? (size_t)(gbase + m0) * H : (size_t)m0 * H) + nbase;
    void* yv = g < E ? y_perm : y_shared;
    uint8_t* stg = As0 + G3_EPI_WAVE_B * wave;
    const int rr = lane >> 3, cu = lane & 7;  // read-back: rows rr + 8q, 16-byte unit cu
    auto write_back = [&](int i, int col0, bool f16) {
      __builtin_amdgcn_wave_barrier();
      g3_u32x4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const g3_u32x4*>(stg + (8 * q + rr) * 128 + 16 * (cu ^ rr));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 32 * i + 8 * q + rr;
        if (r >= mv) continue;
        const uint32_t o = (uint32_t)(r * H + col0);
        g3_u32x4* dst = f16 ? reinterpret_cast<g3_u32x4*>((_Float16*)yv + ybase + o + 8 * cu)
                            : reinterpret_cast<g3_u32x4*>((float*)yv + ybase + o + 4 * cu);
        __builtin_nontemporal_store(v[q], dst);
      }
      __builtin_amdgcn_wave_barrier();
    };
    if (y_f16) {
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        if (i >= nrt) break;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float16v& a = acc[i][sub];
            const g3_f16x4 hv = {(_Float16)a[4 * c], (_Float16)a[4 * c + 1], (_Float16)a[4 * c + 2],
                                 (_Float16)a[4 * c + 3]};
            *reinterpret_cast<g3_f16x4*>(stg + ln * 128 + 16 * ((4 * sub + c) ^ (ln & 7)) + 8 * hh) = hv;
          }
        write_back(i, 0, true);
      }
    } else {
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        if (i >= nrt) break;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float16v& a = acc[i][sub];
            const g3_f32x4 fv = {a[4 * c], a[4 * c + 1], a[4 * c + 2], a[4 * c + 3]};
            *reinterpret_cast<g3_f32x4*>(stg + ln * 128 + 16 * ((2 * c + hh) ^ (ln & 7))) = fv;
          }
          write_back(i, 32 * sub, false);
        }
      }
    }
  }
}

template <int QFMT>
static int launch_gemm_t(const uint16_t* x, int T, int H, int F, const int32_t* row_src, const int32_t* offsets,
                         int k, int E, const int32_t* slot_table, int layer, const void* pool, int64_t record_bytes,
                         void* y_perm, void* y_shared, int y_f16, void* ws, hipStream_t st) {
  int32_t* tile_start = (int32_t*)ws;
  int4* tile_info = (int4*)((uint8_t*)ws + moe_gemm_info_offset(E));
  _Float16* h = (_Float16*)((uint8_t*)ws + moe_gemm_h_offset(T, k, E));
  uint16_t* x16 = (uint16_t*)((uint8_t*)ws + moe_gemm_x16_offset(T, k, E, F));
  {
    const size_t n8 = (size_t)T * H / 8;
    const int grid = 1 + (int)std::min<size_t>((n8 + 1023) / 1024, 1024);
    gemm_prepare_kernel<<<grid, 1024, 0, st>>>(offsets, E, T, k, 32 * g3_rt<QFMT>(), tile_start, tile_info,
                                               (const uint4*)x, n8, (uint4*)x16);
  }
  const int max_tiles = moe_gemm_max_tiles(T, k, E);  // bounds the tile count for BM >= MOE_GEMM_BM
  const int nnt_gu = (2 * F + G3_BN - 1) / G3_BN, nnt_d = (H + G3_BN - 1) / G3_BN;
  const int tot_gu = (max_tiles * nnt_gu + 7) / 8 * 8, tot_d = (max_tiles * nnt_d + 7) / 8 * 8;
  gemm3_kernel<QFMT, true><<<tot_gu, 256, 0, st>>>(x16, T, H, F, k, E, row_src, tile_start, tile_info, slot_table,
                                                   layer, (const uint8_t*)pool, record_bytes, h, y_perm, y_shared,
                                                   y_f16, nnt_gu);
  gemm3_kernel<QFMT, false><<<tot_d, 256, 0, st>>>((const uint16_t*)h, T, H, F, k, E, row_src, tile_start, tile_info,
                                                    slot_table, layer, (const uint8_t*)pool, record_bytes, h, y_perm,
                                                    y_shared, y_f16, nnt_d);
  return moe_check_launch("grouped gemm");
}

extern "C" int moe_grouped_gemm_q(const uint16_t* x, int T, int H, int F, const int32_t* row_src,
                                  const int32_t* offsets, int k, int E, const int32_t* slot_table, int layer,
                                  const void* pool, int64_t record_bytes, int qfmt, void* y_perm, void* y_shared,
                                  int y_dtype, void* ws, size_t ws_bytes, void* stream) {
  int rc = moe_check_expert_shapes(H, F, E, k, qfmt, pool, record_bytes, slot_table, layer);
  if (rc) return rc;
  MOE_REQUIRE(y_dtype == MOE_F32 || y_dtype == MOE_F16, MOE_EUNSUPPORTED, "y_dtype=%d must be MOE_F32 or MOE_F16",
              y_dtype);
  MOE_REQUIRE(T >= 0, MOE_ESHAPE, "T=%d must be >= 0", T);
  MOE_REQUIRE(((int64_t)T * k + T) * (int64_t)(H > F ? H : F) < (1ll << 31) * 8ll, MOE_ESHAPE, "T too large");
  MOE_REQUIRE((int64_t)T * k + T < (1ll << 31), MOE_ESHAPE, "T*k too large");
  // the staging loads address the fp16 copies of x and h with 32-bit byte offsets
  MOE_REQUIRE((int64_t)T * H * 2 < (1ll << 32) && ((int64_t)T * k + T) * F * 2 < (1ll << 32), MOE_ESHAPE,
              "T=%d too large: T*H and (T*k+T)*F fp16 values must stay below 4 GiB", T);
  if (T == 0) return MOE_OK;
  MOE_REQUIRE(x && row_src && offsets && y_perm && y_shared, MOE_EINVAL,
              "x, row_src, offsets, y_perm and y_shared are required");
  MOE_REQUIRE(moe_aligned(x, 16) && moe_aligned(y_perm, 16) && moe_aligned(y_shared, 16), MOE_EALIGN,
              "x, y_perm and y_shared must be 16-byte aligned");
  const size_t need = moe_ws_gemm(T, k, E, H, F);
  MOE_REQUIRE(ws && ws_bytes >= need && moe_aligned(ws, 256), MOE_EWORKSPACE,
              "ws needs %zu bytes, 256-byte aligned", need);
  hipStream_t st = moe_stream(stream);
  const int y_f16 = y_dtype == MOE_F16;
  if (qfmt == MOE_Q4_B32)
    return launch_gemm_t<MOE_Q4_B32>(x, T, H, F, row_src, offsets, k, E, slot_table, layer, pool, record_bytes,
                                     y_perm, y_shared, y_f16, ws, st);
  return launch_gemm_t<MOE_Q2_B16>(x, T, H, F, row_src, offsets, k, E, slot_table, layer, pool, record_bytes, y_perm,
                                   y_shared, y_f16, ws, st);
}
