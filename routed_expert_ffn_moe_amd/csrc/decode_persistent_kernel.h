// One decode / verify step through L layers as ONE persistent kernel.
//
// Batch-1 decode is a strict dependency chain (router -> top-k -> experts ->
// sum -> next layer; "为什么 Strata 在小显存显卡上这么快", section "一个 token，
// 三路工人"), so per-layer kernel boundaries dominate the step.  Here G
// workgroups (at most one per CU) stay resident for the whole step and hand
// data to each other through tagged words instead of kernel boundaries or
// grid barriers:
//   * a producer writes 64-bit words (tag << 32 | payload) with relaxed
//     agent-scope atomic stores (coherent across XCDs, single-copy atomic);
//   * a consumer polls exactly the words it needs until every tag matches
//     the current layer's tag (tags are never reused on a workspace: see
//     the set-up kernels in decode_persistent.hip).  No counters, so nothing
//     serialises.
// Per layer l (tag t_l), workgroup g:
//   A  read x_l (tagged, or x_in for l = 0); 1/rms per token in every wave;
//      router rows e = g (mod G): logits of xn = x * inv, tagged.  Prepare
//      xn for the expert dot products (fp16 pairs) in LDS.
//   B  read all logits; top-k per token (one wave per token: a ballot
//      threshold, then exact ranking of the candidates); with several
//      tokens, the plan of distinct experts (computed identically by every
//      workgroup).  The experts' work is cut into groups of 4 pieces of 8 f
//      values (64 gate/up rows and one down block column each; see "work
//      pieces"), handed out to the workgroups; a group's gate/up dots, SiLU
//      and down dots give a weighted partial output vector of H rows per
//      token, tagged.
//   C  rows r of workgroup g: x_{l+1}[r] = x_l[r] + the G partials, summed
//      in a fixed order.
// Every workgroup produces router rows in A and output rows in C, so no
// workgroup can fall a layer behind the data it still has to read.
// Every wait is bounded; on timeout the error word is set, x_out is filled
// with NaN and the kernel ends.
#pragma once
#include "moe_common.h"
#include "moe_sizes.h"
#include "moe_kernels.h"
#include "moe_topk.h"

#define PT_THREADS 512
#define PT_WAVES 8
#define PT_SPIN_MAX (1 << 18)
#define PT_GROUP_BASE 4  // cost of a group's loads, in units of one token's dot passes
#define PT_MAGIC 0x4d6f4531u
#define PT_CHECK 0x9e3779b9u
// The broadcasts (x, logits) are written once per XCD and each workgroup
// polls its own XCD's copy: a line then has the 32 workgroups of one XCD as
// readers instead of all 256, which shortens an all-to-all hand-off by
// about 0.1 us (x) and 0.5 us (logits) in an exchange microbenchmark.
#define PT_REPL 8
#define PT_EPS 1e-6f

typedef unsigned long long u64;

struct PtArgs {
  const float* x_in;
  int T, H, F, E, k, L, qfmt;
  const uint16_t* w_router;
  const float* bias;
  const int32_t* slot_table;
  const uint8_t* pool;
  int64_t record_bytes;
  float* x_out;
  int32_t* topk_idx_out;
  float* topk_w_out;
  float* x_hist;
  uint32_t* hdr;  // [0] magic, [1] tags reserved, [2] error, [3] check of [1], [4] this call's tag base
  u64* xbuf;      // [PT_REPL][T][H]
  u64* lbuf;      // [PT_REPL][T][E]
  u64* pbuf;      // [(unit * T + i)][H]
  int G, nfs, rpw, tpo;
  size_t prep_bytes;
  unsigned long long* stamps;  // phase timestamps (builds with MOE_PT_STAMPS only), else unused
};

// Phase timestamps for performance analysis: with MOE_PT_STAMPS defined,
// thread 0 of each workgroup records the 100 MHz wall clock at the phase
// boundaries of layers < 64 in LDS (a global store would be counted by the
// next wait for loads, which then also waits for the store) and copies them
// at the end to stamps[(layer * 256 + workgroup) * 16 + i] (PT_MARK stores
// a value there instead of the clock); otherwise the macros are empty.
#ifdef MOE_PT_STAMPS
#define PT_STAMP_DECL __shared__ unsigned long long pt_stamp_lds[64 * 16]
#define PT_STAMP(i)                                                                 \
  do {                                                                              \
    if (threadIdx.x == 0 && l < 64) pt_stamp_lds[l * 16 + (i)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#define PT_MARK(i, v)                                                               \
  do {                                                                              \
    if (threadIdx.x == 0 && l < 64) pt_stamp_lds[l * 16 + (i)] = (unsigned long long)(v); \
  } while (0)
#define PT_STAMP_FLUSH()                                                            \
  do {                                                                              \
    if (threadIdx.x == 0 && blockIdx.x < 256 && a.stamps)                           \
      for (int ls = 0; ls < 64 * 16 && ls < a.L * 16; ++ls)                         \
        a.stamps[((size_t)(ls >> 4) * 256 + blockIdx.x) * 16 + (ls & 15)] = pt_stamp_lds[ls]; \
  } while (0)
#else
#define PT_STAMP_DECL
#define PT_STAMP(i) \
  do {              \
  } while (0)
#define PT_MARK(i, v) \
  do {                \
  } while (0)
#define PT_STAMP_FLUSH() \
  do {                   \
  } while (0)
#endif

__device__ __forceinline__ void pt_put(u64* p, uint32_t tag, float v) {
  __hip_atomic_store(p, ((u64)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool pt_get(const u64* p, uint32_t tag, float& v) {
  const u64 w = __hip_atomic_load(const_cast<u64*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v = __uint_as_float((uint32_t)w);
  return (uint32_t)(w >> 32) == tag;
}
// word `i` of a tagged buffer through a 32-bit byte offset (buffers < 4 GiB),
// so that the address is a uniform base plus a 32-bit lane offset
__device__ __forceinline__ u64* pt_at(u64* base, uint32_t i) {
  return (u64*)((uint8_t*)base + (i << 3));
}
__device__ __forceinline__ u64 pt_load(u64* base, uint32_t i) {
  return __hip_atomic_load(pt_at(base, i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The XCD this workgroup runs on (0..7 on MI355X): selects the copy of a
// broadcast it polls.  Any value would be correct (every copy holds the same
// words); the own XCD's copy only spreads the readers.
__device__ __forceinline__ int pt_xcc() {
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & (PT_REPL - 1);  // HW_REG_XCC_ID[3:0]
}
// Sum over the wave's 64 lanes, returned in every lane: sums over 16, 8, 4
// and 2 lanes inside each row of 16 with DPP row shifts (lane 15 of a row
// then holds the row's sum), rows 0 + 1 and 2 + 3 with row_bcast:15, and the
// two halves with row_bcast:31 (lane 63 then holds the total), which is read
// back as a scalar.  VALU operations with a lane-shift modifier, where a
// butterfly of shuffles takes a round trip through the LDS crossbar per step.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float pt_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, true));
}
__device__ __forceinline__ float pt_wave_sum(float v) {
  v += pt_dpp<0x111, 0xf>(v);  // row_shr:1
  v += pt_dpp<0x112, 0xf>(v);  // row_shr:2
  v += pt_dpp<0x114, 0xf>(v);  // row_shr:4
  v += pt_dpp<0x118, 0xf>(v);  // row_shr:8
  v += pt_dpp<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += pt_dpp<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// Inclusive prefix sum over the wave's 64 lanes (integers): within each row
// of 16 with row shifts of 1, 2, 4, 8, then rows 1 and 3 add lane 15 of rows
// 0 and 2 (row_bcast:15), and rows 2 and 3 add lane 31 (row_bcast:31).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int pt_dppi(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, true);
}
__device__ __forceinline__ int pt_wave_scan(int v) {
  v += pt_dppi<0x111, 0xf>(v);
  v += pt_dppi<0x112, 0xf>(v);
  v += pt_dppi<0x114, 0xf>(v);
  v += pt_dppi<0x118, 0xf>(v);
  v += pt_dppi<0x142, 0xa>(v);
  v += pt_dppi<0x143, 0xc>(v);
  return v;
}
// The value of lane l ^ 1 and of lane l ^ 2 (DPP quad permutes), and of lane
// l + 4 inside the lane's row of 16 (0 past the row's end).
__device__ __forceinline__ float pt_xor1(float v) { return pt_dpp<0xB1, 0xf>(v); }
__device__ __forceinline__ float pt_xor2(float v) { return pt_dpp<0x4E, 0xf>(v); }
__device__ __forceinline__ float pt_next4(float v) { return pt_dpp<0x104, 0xf>(v); }
// Sums over aligned segments of n lanes (n a power of two <= 32), left in the
// segment's last lane: running sums over 2, 4, 8, 16 lanes with row shifts,
// and for n = 32 the two rows of each half joined with row_bcast:15.
__device__ __forceinline__ float pt_segment_sum(float v, int n) {
  if (n > 1) v += pt_dpp<0x111, 0xf>(v);   // row_shr:1
  if (n > 2) v += pt_dpp<0x112, 0xf>(v);   // row_shr:2
  if (n > 4) v += pt_dpp<0x114, 0xf>(v);   // row_shr:4
  if (n > 8) v += pt_dpp<0x118, 0xf>(v);   // row_shr:8
  if (n > 16) v += pt_dpp<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  return v;
}

// The thread index and lane, made opaque at each call: values derived from
// them inside the layer loop are then computed where used instead of being
// hoisted out of the loop and kept live (or spilled) for the whole kernel.
__device__ __forceinline__ int pt_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}
__device__ __forceinline__ int pt_lane() { return pt_tid() & 63; }

// Polling: each thread reloads its own words until they all carry the tag,
// with no sleep and no workgroup barrier between rounds; one barrier
// follows.  In an exchange microbenchmark (256 workgroups, one per
// CU) this took an all-to-all hand-off from 2.9 to 2.1 us (x, 2,048 words),
// 2.5 to 2.3 us (logits, 512 words) and 4.3 to 3.4-3.6 us (partial sums,
// 8 rows of 256 producers) against polling in lock-step with a barrier per
// round; a sleep between rounds only delayed the detection.
// Polls words base[off + tid + PT_THREADS q] (q < NQ, indices past `last`
// clamped to it) until every one carries `tag`; w receives them.  SPARSE:
// reload only the words still missing (fewer loads per round, but the
// per-word state costs registers), else reload all of them each round.
// Returns false on timeout.  Per thread, no barrier.
template <int NQ, bool SPARSE>
__device__ __forceinline__ bool pt_poll(u64 (&w)[NQ], u64* base, uint32_t off, int tid, int last, uint32_t tag) {
  if (SPARSE) {
    bool need[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) need[q] = true;
    for (int it = 0;; ++it) {
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if (need[q]) w[q] = pt_load(base, off + (uint32_t)min(tid + q * PT_THREADS, last));
      bool any = false;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        need[q] = need[q] && (uint32_t)(w[q] >> 32) != tag;
        any |= need[q];
      }
      if (!any) return true;
      if (it > PT_SPIN_MAX) return false;
    }
  }
  for (int it = 0;; ++it) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) w[q] = pt_load(base, off + (uint32_t)min(tid + q * PT_THREADS, last));
    bool mine = true;
#pragma unroll
    for (int q = 0; q < NQ; ++q) mine &= (uint32_t)(w[q] >> 32) == tag;
    if (mine) return true;
    if (it > PT_SPIN_MAX) return false;
  }
}

// tag of layer l of the call whose tags start after `base`
__device__ __forceinline__ uint32_t pt_tag(uint32_t base, int l) { return base + (uint32_t)l + 1u; }

// ---------------------------------------------------------------- small helpers
// The nibble / crumb masks of the dots, held in registers (made opaque once
// per layer): (x & mask) | magic is then one v_and_or_b32; with both
// operands literal constants it takes two instructions, as the VOP3
// encoding takes no literal here.  int4: q = 0x000F000F, r = 0x00F000F0;
// int2: q, r, s, t = 0x00030003 << 2i.
struct PtMask {
  uint32_t q, r, s, t;
};
__device__ __forceinline__ PtMask pt_masks(int qfmt) {
  PtMask m;
  if (qfmt == MOE_Q4_B32) {
    m.q = 0x000F000Fu; m.r = 0x00F000F0u; m.s = 0u; m.t = 0u;
  } else {
    m.q = 0x00030003u; m.r = 0x000C000Cu; m.s = 0x00300030u; m.t = 0x00C000C0u;
  }
  asm volatile("" : "+v"(m.q), "+v"(m.r), "+v"(m.s), "+v"(m.t));
  return m;
}
// dot of one int4 block (16 bytes) with a prepared activation block
__device__ __forceinline__ float pt_q4_dot(uint4 q, const uint32_t* xp, float c, const PtMask& mk) {
  const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
  float d = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = qw[j], w8 = qw[j] >> 8;
    d = moe_dot2(moe_u32_as_half2((w & mk.q) | MOE_F16_1024X2), moe_u32_as_half2(xp[4 * j + 0]), d);
    d = moe_dot2(moe_u32_as_half2((w & mk.r) | MOE_F16_1024X2), moe_u32_as_half2(xp[4 * j + 1]), d);
    d = moe_dot2(moe_u32_as_half2((w8 & mk.q) | MOE_F16_1024X2), moe_u32_as_half2(xp[4 * j + 2]), d);
    d = moe_dot2(moe_u32_as_half2((w8 & mk.r) | MOE_F16_1024X2), moe_u32_as_half2(xp[4 * j + 3]), d);
  }
  return d - c;
}
// one int2 block (one word) with a prepared block: s * (dot - c0) + m * sum(x)
__device__ __forceinline__ float pt_q2_dot(uint32_t w, float s, float m, const uint32_t* xp, float2 c, const PtMask& mk) {
  const uint32_t w8 = w >> 8;
  float d = 0.f;
  d = moe_dot2(moe_u32_as_half2((w & mk.q) | MOE_F16_1024X2), moe_u32_as_half2(xp[0]), d);
  d = moe_dot2(moe_u32_as_half2((w & mk.r) | MOE_F16_1024X2), moe_u32_as_half2(xp[1]), d);
  d = moe_dot2(moe_u32_as_half2((w & mk.s) | MOE_F16_1024X2), moe_u32_as_half2(xp[2]), d);
  d = moe_dot2(moe_u32_as_half2((w & mk.t) | MOE_F16_1024X2), moe_u32_as_half2(xp[3]), d);
  d = moe_dot2(moe_u32_as_half2((w8 & mk.q) | MOE_F16_1024X2), moe_u32_as_half2(xp[4]), d);
  d = moe_dot2(moe_u32_as_half2((w8 & mk.r) | MOE_F16_1024X2), moe_u32_as_half2(xp[5]), d);
  d = moe_dot2(moe_u32_as_half2((w8 & mk.s) | MOE_F16_1024X2), moe_u32_as_half2(xp[6]), d);
  d = moe_dot2(moe_u32_as_half2((w8 & mk.t) | MOE_F16_1024X2), moe_u32_as_half2(xp[7]), d);
  return fmaf(s, d - c.x, m * c.y);
}

// dot of one int4 word (8 values) with its prepared activations xp[4]
__device__ __forceinline__ float pt_q4_word(uint32_t w, const uint32_t* xp, float c, const PtMask& mk) {
  const uint32_t w8 = w >> 8;
  float d = 0.f;
  d = moe_dot2(moe_u32_as_half2((w & mk.q) | MOE_F16_1024X2), moe_u32_as_half2(xp[0]), d);
  d = moe_dot2(moe_u32_as_half2((w & mk.r) | MOE_F16_1024X2), moe_u32_as_half2(xp[1]), d);
  d = moe_dot2(moe_u32_as_half2((w8 & mk.q) | MOE_F16_1024X2), moe_u32_as_half2(xp[2]), d);
  d = moe_dot2(moe_u32_as_half2((w8 & mk.r) | MOE_F16_1024X2), moe_u32_as_half2(xp[3]), d);
  return d - c;
}
// 8 values of an int2 block word (the low or high byte of each half, w
// already shifted): s * (dot - c0) + m * sum(x)
__device__ __forceinline__ float pt_q2_word(uint32_t w, float s, float m, const uint32_t* xp, float2 c, const PtMask& mk) {
  float d = 0.f;
  d = moe_dot2(moe_u32_as_half2((w & mk.q) | MOE_F16_1024X2), moe_u32_as_half2(xp[0]), d);
  d = moe_dot2(moe_u32_as_half2((w & mk.r) | MOE_F16_1024X2), moe_u32_as_half2(xp[1]), d);
  d = moe_dot2(moe_u32_as_half2((w & mk.s) | MOE_F16_1024X2), moe_u32_as_half2(xp[2]), d);
  d = moe_dot2(moe_u32_as_half2((w & mk.t) | MOE_F16_1024X2), moe_u32_as_half2(xp[3]), d);
  return fmaf(s, d - c.x, m * c.y);
}

// Prepared block writers (same arithmetic as the standalone decode path).
template <int QFMT>
__device__ void pt_prep_block(const float* b, float scale, uint32_t* p, float2* corr) {
  if (QFMT == MOE_Q4_B32) {
    const half2v k0 = {(_Float16)1032.f, (_Float16)1032.f};
    const half2v k1 = {(_Float16)1152.f, (_Float16)1152.f};
    float c = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half2v a0 = {(_Float16)(b[8 * j + 0] * scale), (_Float16)(b[8 * j + 1] * scale)};
      half2v a1 = {(_Float16)(b[8 * j + 2] * scale * 0.0625f), (_Float16)(b[8 * j + 3] * scale * 0.0625f)};
      half2v a2 = {(_Float16)(b[8 * j + 4] * scale), (_Float16)(b[8 * j + 5] * scale)};
      half2v a3 = {(_Float16)(b[8 * j + 6] * scale * 0.0625f), (_Float16)(b[8 * j + 7] * scale * 0.0625f)};
      p[4 * j + 0] = moe_half2_as_u32(a0);
      p[4 * j + 1] = moe_half2_as_u32(a1);
      p[4 * j + 2] = moe_half2_as_u32(a2);
      p[4 * j + 3] = moe_half2_as_u32(a3);
      c = moe_dot2(a0, k0, c);
      c = moe_dot2(a1, k1, c);
      c = moe_dot2(a2, k0, c);
      c = moe_dot2(a3, k1, c);
    }
    *corr = make_float2(c, 0.f);
  } else {
    const half2v k1024 = {(_Float16)1024.f, (_Float16)1024.f};
    float c0 = 0.f, sx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float mul = (i & 3) == 0 ? 1.f : (i & 3) == 1 ? 0.25f : (i & 3) == 2 ? 0.0625f : 0.015625f;
      half2v a = {(_Float16)(b[2 * i] * scale * mul), (_Float16)(b[2 * i + 1] * scale * mul)};
      p[i] = moe_half2_as_u32(a);
      const half2v kc = {(_Float16)(1.f / mul), (_Float16)(1.f / mul)};
      c0 = moe_dot2(a, k1024, c0);
      sx = moe_dot2(a, kc, sx);
    }
    *corr = make_float2(c0, sx);
  }
}

// Work plan of one layer from the T * k chosen experts (one wave): the
// distinct experts ("units") in order of first occurrence (token-major), each
// with its tokens p_tok[ts u + c] and their top-k positions p_j[ts u + c]
// (ts >= T: a unit holds each token at most once);
// then, if with_shared, the shared expert with every token (top-k position
// k); p_roff[u] is the byte offset of the unit's record in the pool;
// p_misc[0] = the number of units.  n = T * k <= 128.  scr_mask, scr_unit:
// LDS scratch of E entries each.
__device__ __forceinline__ void pt_plan(const int* topi, int T, int k, int E, const int32_t* slots, int64_t rbytes,
                                        bool with_shared, int ts, int* p_exp, int* p_ntok, int* p_tok, int* p_j,
                                        int64_t* p_roff, int* p_cum, int* p_misc, uint32_t* scr_mask,
                                        int* scr_unit) {
  const int lane = pt_lane(), n = T * k;
  if (T == 1) {  // one token: its k experts are distinct, in top-k order
    if (lane < k) {
      const int e1 = topi[lane];
      p_exp[lane] = e1;
      p_ntok[lane] = 1;
      p_roff[lane] = (int64_t)slots[e1] * rbytes;
      p_tok[lane * ts] = 0;
      p_j[lane * ts] = lane;
    }
    if (lane == 0) {
      if (with_shared) {
        p_exp[k] = E;
        p_ntok[k] = 1;
        p_roff[k] = (int64_t)slots[E] * rbytes;
        p_tok[k * ts] = 0;
        p_j[k * ts] = k;
      }
      p_misc[0] = with_shared ? k + 1 : k;
    }
    return;
  }
  // Entry i = (token t, position j), i < n <= 128: lane l holds entries l
  // and l + 64.  A token's k experts are distinct, so per expert the bitmask
  // of the tokens that chose it (scr_mask[e], cleared first by the lanes that
  // use it, then OR-ed) gives each entry the number of earlier tokens with the
  // same expert (`before`: its place in the unit's token list), the expert's
  // token count, and whether the entry is the expert's first occurrence
  // (before == 0).  The units are numbered by their first occurrences in
  // entry order; scr_unit[e] hands the number to the other entries of the
  // expert.
  bool act[2];
  int tv[2], jv[2], ev[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int i = lane + 64 * r;
    act[r] = i < n;
    tv[r] = act[r] ? i / k : 0;
    jv[r] = act[r] ? i - tv[r] * k : 0;
    ev[r] = act[r] ? topi[i] : 0;
  }
#pragma unroll
  for (int r = 0; r < 2; ++r)
    if (act[r]) scr_mask[ev[r]] = 0u;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int r = 0; r < 2; ++r)
    if (act[r]) __hip_atomic_fetch_or(scr_mask + ev[r], 1u << tv[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  int before[2];
  uint64_t firsts[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint32_t msk = act[r] ? scr_mask[ev[r]] : 0u;
    before[r] = (int)__popc(msk & ((1u << tv[r]) - 1u));
    firsts[r] = __ballot(act[r] && before[r] == 0);
  }
  const int U0 = (int)__popcll(firsts[0]), U = U0 + (int)__popcll(firsts[1]);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (act[r] && before[r] == 0) {
      const int u = (r == 0 ? 0 : U0) + (int)__popcll(firsts[r] & ((1ull << lane) - 1ull));  // rank among first occurrences
      scr_unit[ev[r]] = u;
      p_exp[u] = ev[r];
      p_ntok[u] = (int)__popc(scr_mask[ev[r]]);
      p_roff[u] = (int64_t)slots[ev[r]] * rbytes;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (act[r]) {
      const int u = scr_unit[ev[r]];
      p_tok[u * ts + before[r]] = tv[r];
      p_j[u * ts + before[r]] = jv[r];
    }
  }
  if (with_shared) {
    if (lane < T) {
      p_tok[U * ts + lane] = lane;
      p_j[U * ts + lane] = k;
    }
    if (lane == 0) {
      p_exp[U] = E;
      p_ntok[U] = T;
      p_roff[U] = (int64_t)slots[E] * rbytes;
    }
  }
  // p_cum[u] = the summed costs of units < u, a group of unit u costing
  // PT_GROUP_BASE + (its token count); p_cum[U1] = all of them
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const int c0 = lane < U ? PT_GROUP_BASE + p_ntok[lane] : 0;
  const int c1 = lane + 64 < U ? PT_GROUP_BASE + p_ntok[lane + 64] : 0;
  const int incl0 = pt_wave_scan(c0);
  const int incl1 = pt_wave_scan(c1) + __builtin_amdgcn_readlane(incl0, 63);
  if (lane < U) p_cum[lane] = incl0 - c0;
  if (lane + 64 < U) p_cum[lane + 64] = incl1 - c1;
  const int sum_r = U == 0 ? 0 : U <= 64 ? __builtin_amdgcn_readlane(incl0, U - 1) : __builtin_amdgcn_readlane(incl1, U - 65);
  if (lane == 0) {
    p_cum[U] = sum_r;
    if (with_shared) p_cum[U + 1] = sum_r + PT_GROUP_BASE + T;
    p_misc[0] = with_shared ? U + 1 : U;
  }
}

// Prepared activations, one 8-value word of a quantisation block per thread.
// int4: 4 threads per 32-value block; int2: 2 threads per 16-value block.
// The block correction is summed over those lanes with shuffles (the lanes
// of a block are consecutive and the shuffles are executed by the whole wave).
template <int QFMT>
__device__ __forceinline__ void pt_prep_word(const float* v, float scale, bool valid, uint32_t* p, float2* corr,
                                             int sub) {
  float c0 = 0.f, c1 = 0.f;
  if (QFMT == MOE_Q4_B32) {
    const half2v k0 = {(_Float16)1032.f, (_Float16)1032.f};
    const half2v k1 = {(_Float16)1152.f, (_Float16)1152.f};
    if (valid) {
      half2v a0 = {(_Float16)(v[0] * scale), (_Float16)(v[1] * scale)};
      half2v a1 = {(_Float16)(v[2] * scale * 0.0625f), (_Float16)(v[3] * scale * 0.0625f)};
      half2v a2 = {(_Float16)(v[4] * scale), (_Float16)(v[5] * scale)};
      half2v a3 = {(_Float16)(v[6] * scale * 0.0625f), (_Float16)(v[7] * scale * 0.0625f)};
      p[0] = moe_half2_as_u32(a0);
      p[1] = moe_half2_as_u32(a1);
      p[2] = moe_half2_as_u32(a2);
      p[3] = moe_half2_as_u32(a3);
      c0 = moe_dot2(a0, k0, c0);
      c0 = moe_dot2(a1, k1, c0);
      c0 = moe_dot2(a2, k0, c0);
      c0 = moe_dot2(a3, k1, c0);
    }
    c0 += pt_xor1(c0);
    c0 += pt_xor2(c0);
    if (valid && sub == 0) *corr = make_float2(c0, 0.f);
  } else {
    const half2v k1024 = {(_Float16)1024.f, (_Float16)1024.f};
    if (valid) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // pairs 4*sub + i of the block: multiplier 4^i
        const float mul = i == 0 ? 1.f : i == 1 ? 0.25f : i == 2 ? 0.0625f : 0.015625f;
        half2v a = {(_Float16)(v[2 * i] * scale * mul), (_Float16)(v[2 * i + 1] * scale * mul)};
        p[i] = moe_half2_as_u32(a);
        const half2v kc = {(_Float16)(1.f / mul), (_Float16)(1.f / mul)};
        c0 = moe_dot2(a, k1024, c0);
        c1 = moe_dot2(a, kc, c1);
      }
    }
    c0 += pt_xor1(c0);
    c1 += pt_xor1(c1);
    if (valid && sub == 0) *corr = make_float2(c0, c1);
  }
}

// ---------------------------------------------------------------- LDS layout
// Section offsets (bytes, 16-byte aligned) shared by the kernel and the host.
struct PtLds {
  size_t xs, xprep, lg, topi, topw, p_exp, p_ntok, p_tok, p_j, p_roff, p_cum, p_misc, red, hp, hc, slots, ss, total;
};
#define PT_PB_MAX 5    // pieces per batch: 4 of row slot A, 1 of row slot B
#define PT_SLOTS 80    // gate/up row slots per batch (16 per piece)
// Token slots the layout provides for T tokens (at least the MT of the
// instance that runs them: 4 up to 4 tokens, 8 above), which is also the
// per-unit token stride of the plan.
__host__ __device__ inline int pt_token_slots(int T) { return T <= 4 ? 4 : 8; }
__host__ __device__ inline PtLds pt_lds(int qfmt, int T, int k, int E, int H, size_t prep_bytes) {
  PtLds o;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = (off + bytes + 15) / 16 * 16;
    return at;
  };
  const size_t U1max = (size_t)T * k + 1;
  const size_t ts = (size_t)pt_token_slots(T);
  (void)qfmt;
  o.xs = take((size_t)T * H * 4);
  o.xprep = take((size_t)T * prep_bytes);
  o.lg = take((size_t)T * E * 4);
  o.topi = take((size_t)T * k * 4);
  o.topw = take((size_t)T * k * 4);
  o.p_exp = take(U1max * 4);
  o.p_ntok = take(U1max * 4);
  o.p_tok = take(U1max * ts * 4);
  o.p_j = take(U1max * ts * 4);
  o.p_roff = take(U1max * 8);
  o.p_cum = take((U1max + 1) * 4);
  o.p_misc = take(16);
  o.red = take((size_t)PT_WAVES * PT_SLOTS * ts * 4);  // [wave][slot][token slot] partial gate/up dots
  o.hp = take((size_t)PT_PB_MAX * ts * 4 * 4);         // [piece][token slot][4] prepared h words
  o.hc = take((size_t)PT_PB_MAX * ts * 8);             // [piece][token slot] corrections
  o.slots = take((size_t)(E + 1) * 4);
  o.ss = take((size_t)PT_WAVES * 8 * 4);  // [wave][token slot] sums of squares
  o.total = off;
  return o;
}

// ---------------------------------------------------------------- the kernel
template <int QFMT, int MT, int SLOTS>
__global__ __launch_bounds__(PT_THREADS) void decode_persistent_kernel(PtArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  PT_STAMP_DECL;
  const int T = a.T, H = a.H, F = a.F, E = a.E, k = a.k, L = a.L, G = a.G;
  const int g = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  int tid = threadIdx.x, lane = tid & 63;
  const int blk = QFMT == MOE_Q4_B32 ? 32 : 16;
  const MoePlanes pl = moe_planes(QFMT, H, F);  // a record is < 4 GiB: 32-bit plane offsets
  const uint32_t o_guq = (uint32_t)pl.gu_q, o_gus = (uint32_t)pl.gu_s, o_dq = (uint32_t)pl.d_q, o_ds = (uint32_t)pl.d_s;

  const PtLds o = pt_lds(QFMT, T, k, E, H, a.prep_bytes);
  float* xs = (float*)(smem + o.xs);          // [T][H]
  uint8_t* xprep = smem + o.xprep;            // [T][prep_bytes]
  float* lg = (float*)(smem + o.lg);          // [T][E]
  int* topi = (int*)(smem + o.topi);          // [T][k]
  float* topw = (float*)(smem + o.topw);      // [T][k]
  int* p_exp = (int*)(smem + o.p_exp);        // [U1max]
  int* p_ntok = (int*)(smem + o.p_ntok);      // [U1max]
  constexpr int TS = MT > 4 ? 8 : 4;          // per-unit token stride of the plan
  int* p_tok = (int*)(smem + o.p_tok);        // [U1max][TS]
  int* p_j = (int*)(smem + o.p_j);            // [U1max][TS]
  int64_t* p_roff = (int64_t*)(smem + o.p_roff); // [U1max] record byte offsets
  int* p_cum = (int*)(smem + o.p_cum);        // [U1max + 1] group cost prefix per unit
  int* p_misc = (int*)(smem + o.p_misc);      // [0] = U1
  float* red = (float*)(smem + o.red);        // [wave][slot][MT]
  uint32_t* hp = (uint32_t*)(smem + o.hp);    // [piece][MT][4]
  float2* hc = (float2*)(smem + o.hc);        // [piece][MT]
  int* lslots = (int*)(smem + o.slots);        // [E+1] this layer's slot-table row
  float* ssred = (float*)(smem + o.ss);        // [wave][MT] per-wave sums of squares of x_l

  const uint32_t base = __hip_atomic_load(a.hdr + 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  bool ok = true;
  const int nrch = (H + 511) / 512;  // router chunks of 512 columns per row (<= 4)
  const float inv_h = 1.0f / (float)H;

  for (int l = 0; l < L && ok; ++l) {
    // the thread index is made opaque once per layer, so that the compiler
    // derives per-thread offsets where they are used instead of keeping them
    // live across the whole layer loop
    asm volatile("" : "+v"(tid));
    lane = tid & 63;
    const uint32_t tag = pt_tag(base, l);
    PT_STAMP(0);
    // ------------------------------------------------------------ phase A
    // this wave's router row (if any) is requested before waiting for x_l
    // (indices are clamped into range so that every load is unconditional)
    // this layer's slot-table row (E + 1 <= 1025 entries, <= 3 per thread),
    // requested now and kept in LDS for the plan
    int srow[3];
#pragma unroll
    for (int c = 0; c < 3; ++c)
      srow[c] = a.slot_table[(size_t)l * (E + 1) + min(tid + PT_THREADS * c, E)];
    const uint16_t* wr = a.w_router + (size_t)l * E * H;  // wave-uniform; 32-bit offsets below
    // Router work of this workgroup: its rows e = g + G r (nrow of them) for
    // each of the T tokens, as items i = t * nrow + r spread over the waves
    // (wave w takes items w, w + 8, ...); each item is one token's dot
    // product with one row.  The row of the wave's first item is requested
    // here, before waiting for x_l.
    const int nrow = (E - g + G - 1) / G;
    const int nitem = T * nrow;
    const int e_row = g + G * (wave % nrow);
    // its routing bias too (a load issued only after the dot product would
    // put a memory round trip between x's arrival and the published logit)
    const float b_row = a.bias ? a.bias[(size_t)l * E + min(e_row, E - 1)] : 0.f;
    uint4 rw[4];
    if (wave < nitem) {  // wave-uniform
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t h0 = 512 * c + 8 * lane;
        rw[c] = *reinterpret_cast<const uint4*>(wr + (uint32_t)e_row * (uint32_t)H + (h0 < (uint32_t)H ? h0 : 0u));
      }
    }
    // Work is handed out in groups of 4 pieces (see "work pieces" below).  One
    // token: when the units' groups outnumber the workgroups by at most G/4,
    // every workgroup takes one group and the remaining groups (the last ones
    // of the shared expert) are split into single pieces, one per workgroup at
    // most.  Such a piece's gate/up rows and down words are requested here,
    // before x_l and the logits are exchanged, and used as row slot B (piece
    // 4) of the batch.  Row slot B: gate/up row l % 16 of the piece over a
    // quarter of the wave's K range (lane group l / 16).
    const int NP = F / 8;
    const int NKU = H / 128;                                     // K units of 128 values
    const int ku0 = wave * NKU / 8, ku1 = (wave + 1) * NKU / 8;  // <= 2 per wave
    const int lq = lane >> 4;
    const int kuB = min(ku0 + (lq >> 1), NKU - 1);
    const bool kvB = ku0 + (lq >> 1) < ku1;
    const int TG1 = (k + 1) * (NP / 4);  // groups with one token: k experts and the shared one
    const int nL = 4 * (TG1 - G);        // single pieces left over
    const bool sepB = MT == 1 && nL > 0 && nL <= NP && nL <= G;
    int sp = -1;  // this workgroup's single shared piece
    if (sepB) {
      const int j0 = (int)((int64_t)g * nL / G), j1 = (int)((int64_t)(g + 1) * nL / G);
      sp = j1 > j0 ? NP - nL + j0 : -1;
    }
    uint4 gqS[2] = {};
    uint32_t gsS = 0u;
    uint32_t dwS[4] = {0u, 0u, 0u, 0u}, dmS[4] = {0u, 0u, 0u, 0u};
    if (sp >= 0) {  // uniform over the workgroup
      const uint8_t* recS = a.pool + (int64_t)a.slot_table[(size_t)l * (E + 1) + E] * a.record_bytes;
      const int i = lane & 15;
      const uint32_t rowS = (uint32_t)(64 * (sp >> 2) + 8 * (sp & 3) + (i & 7) + (i >= 8 ? 32 : 0));
      if (QFMT == MOE_Q4_B32) {
        const uint32_t kb0 = 4u * kuB + 2u * (lq & 1);
        gsS = *reinterpret_cast<const uint32_t*>(recS + (o_gus + 16u * (uint32_t)kuB * (uint32_t)F + 8u * rowS + 4u * (lq & 1)));
#pragma unroll
        for (int b = 0; b < 2; ++b)
          gqS[b] = *reinterpret_cast<const uint4*>(recS + (o_guq + 16u * ((kb0 + b) * 2u * (uint32_t)F + rowS)));
      } else {
        const uint32_t un = 2u * kuB + (lq & 1);
        gqS[0] = *reinterpret_cast<const uint4*>(recS + (o_guq + 16u * (un * 2u * (uint32_t)F + rowS)));
        gqS[1] = *reinterpret_cast<const uint4*>(recS + (o_gus + 16u * (un * 2u * (uint32_t)F + rowS)));
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t r = (uint32_t)min(tid + 512 * c, H - 1);
        if (QFMT == MOE_Q4_B32) {
          const uint32_t bc = (uint32_t)(sp >> 2);
          dwS[c] = *reinterpret_cast<const uint32_t*>(recS + (o_dq + 16u * (bc * (uint32_t)H + r) + 4u * (sp & 3)));
          dmS[c] = *reinterpret_cast<const uint16_t*>(recS + (o_ds + 2u * (bc * (uint32_t)H + r)));
        } else {
          const uint32_t b2 = (uint32_t)(sp >> 1);
          dwS[c] = *reinterpret_cast<const uint32_t*>(recS + (o_dq + 4u * (b2 * (uint32_t)H + r)));
          dmS[c] = *reinterpret_cast<const uint32_t*>(recS + (o_ds + 4u * (b2 * (uint32_t)H + r)));
        }
      }
    }
    constexpr int NX = 4 * MT;  // words of x per thread: T * H <= 512 * NX
    // x_l into LDS.  One token: each thread also sums the squares of its
    // words (word tid + 512 q in order, then the wave's butterfly), so 1/rms
    // needs no second pass over x.
    float ssq[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) ssq[t] = 0.f;
    // several tokens with H a multiple of 512: word q of a thread belongs to
    // token q / (H / 512), so the squares can be summed from the polled words
    // too, in the same order as the LDS pass below
    const bool ssq_poll = MT == 1 || H % PT_THREADS == 0;
    const int wpt = H / PT_THREADS;  // words of a token per thread (ssq_poll)
    {
      const int last = T * H - 1;
      u64 w[NX];
      if (l == 0) {
#pragma unroll
        for (int q = 0; q < NX; ++q)
          w[q] = (u64)__float_as_uint(a.x_in[min(tid + q * PT_THREADS, last)]);
      } else {
        const uint32_t ptag = pt_tag(base, l - 1);
        const uint32_t xoff = (uint32_t)(pt_xcc() * T * H);
        // each thread polls its own words until they all carry the tag (no
        // workgroup barrier per polling round); pt_poll reloads only the words
        // still missing where registers allow it (one token)
        ok = pt_poll<NX, MT == 1>(w, a.xbuf, xoff, tid, last, ptag);
      }
#pragma unroll
      for (int q = 0; q < NX; ++q) {
        const int i = tid + q * PT_THREADS;
        if (i <= last) {
          const float v = __uint_as_float((uint32_t)w[q]);
          xs[i] = v;
          if (MT == 1) {
            ssq[0] = fmaf(v, v, ssq[0]);
          } else {
#pragma unroll
            for (int t = 0; t < MT; ++t)
              if (q >= t * wpt && q < (t + 1) * wpt) ssq[t] = fmaf(v, v, ssq[t]);
          }
        }
      }
      if (ssq_poll) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const float v = pt_wave_sum(ssq[t]);
          if (lane == 0) ssred[wave * MT + t] = v;
        }
      }
      if (!__syncthreads_and(ok)) { ok = false; break; }
    }
    PT_STAMP(1);  // x_l received
    // 1 / rms of every token: thread tid sums the squares of the token's
    // words tid + 512 q in order, the wave adds its threads (DPP), and the 8
    // waves' sums are added in order.  From the polled words above (no second
    // pass) for one token, and for several when H is a multiple of 512; else
    // from LDS, one more barrier.  The order is the same for every token
    // count, so a token's 1/rms does not depend on the window it is verified in.
    if (!ssq_poll) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        float ss = 0.f;
        if (t < T)
          for (int h = tid; h < H; h += PT_THREADS) ss = fmaf(xs[t * H + h], xs[t * H + h], ss);
        ss = pt_wave_sum(ss);
        if (lane == 0) ssred[wave * MT + t] = ss;
      }
      __syncthreads();
    }
    float invr[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      float ss = 0.f;
#pragma unroll
      for (int w8 = 0; w8 < PT_WAVES; ++w8) ss += ssred[w8 * MT + t];
      invr[t] = __builtin_amdgcn_rsqf(ss * inv_h + PT_EPS);
    }
    PT_STAMP(10);  // 1/rms
    if (a.x_hist && g == 0)
      for (int i = tid; i < T * H; i += PT_THREADS) a.x_hist[(size_t)l * T * H + i] = xs[i];
    // router items of this wave: the prefetched row first, another row only
    // when an item needs one (a wave keeps one row when nrow divides 8)
    {
      int e_cur = e_row;
      float b_cur = b_row;
      for (int i = wave; i < nitem; i += PT_WAVES) {
        const int t = i / nrow, e = g + G * (i % nrow);
        if (e != e_cur) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t h0 = 512 * c + 8 * lane;
            rw[c] = *reinterpret_cast<const uint4*>(wr + (uint32_t)e * (uint32_t)H + (h0 < (uint32_t)H ? h0 : 0u));
          }
          b_cur = a.bias ? a.bias[(size_t)l * E + e] : 0.f;
          e_cur = e;
        }
        const float* xt = xs + (size_t)t * H;
        float accs[4] = {0.f, 0.f, 0.f, 0.f};  // one per chunk: four short FMA chains
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int h0 = 512 * c + 8 * lane;
          if (c < nrch && h0 < H) {
            const uint32_t ww[4] = {rw[c].x, rw[c].y, rw[c].z, rw[c].w};
            const float4 xa = *reinterpret_cast<const float4*>(xt + h0);
            const float4 xb = *reinterpret_cast<const float4*>(xt + h0 + 4);
            const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {  // the 4 words (8 bf16) of the chunk
              accs[c] = fmaf(xv[2 * q], __uint_as_float(ww[q] << 16), accs[c]);
              accs[c] = fmaf(xv[2 * q + 1], __uint_as_float(ww[q] & 0xffff0000u), accs[c]);
            }
          }
        }
        const float acc = (accs[0] + accs[1]) + (accs[2] + accs[3]);
        float it = invr[0];
#pragma unroll
        for (int q = 1; q < MT; ++q) it = t == q ? invr[q] : it;
        const float sdot = pt_wave_sum(acc);
        if (lane < PT_REPL)  // lane r writes the copy of XCD r
          pt_put(pt_at(a.lbuf, (uint32_t)((lane * T + t) * E + e)), tag, sdot * it + b_cur);
      }
    }
    PT_STAMP(11);  // router rows published
    // prepared xn for the gate/up dot products: one 8-value word per thread
    {
      const int nwords = T * H / 8;
      for (int w0 = 0; w0 < nwords; w0 += PT_THREADS) {
        const int wi = w0 + tid;
        const bool valid = wi < nwords;
        const int t = valid ? wi / (H / 8) : 0, wh = valid ? wi % (H / 8) : 0;  // word within the token
        const int b = wh / (blk / 8), sub = wh % (blk / 8);
        uint8_t* out = xprep + (size_t)t * a.prep_bytes;
        float it = invr[0];
#pragma unroll
        for (int q = 1; q < MT; ++q) it = t == q ? invr[q] : it;
        pt_prep_word<QFMT>(xs + (size_t)t * H + 8 * wh, it, valid, (uint32_t*)out + (blk / 2) * b + 4 * sub,
                           (float2*)(out + 2 * (size_t)H) + b, sub);
      }
    }
    PT_STAMP(2);  // x prepared
    // this layer's slot-table row into LDS (made visible by the barrier after
    // the logits arrive)
#pragma unroll
    for (int c = 0; c < 3; ++c)
      if (tid + PT_THREADS * c <= E) lslots[tid + PT_THREADS * c] = srow[c];
    // ------------------------------------------------------------ phase B
    {
      constexpr int NLG = MT * SLOTS / 8 > 0 ? MT * SLOTS / 8 : 1;  // T * E <= 512 * NLG
      const int last = T * E - 1;
      const uint32_t loff = (uint32_t)(pt_xcc() * T * E);
      u64 w[NLG];
      ok = pt_poll<NLG, MT == 1>(w, a.lbuf, loff, tid, last, tag);
#pragma unroll
      for (int q = 0; q < NLG; ++q)
        if (tid + q * PT_THREADS <= last) lg[tid + q * PT_THREADS] = __uint_as_float((uint32_t)w[q]);
    }
    if (!__syncthreads_and(ok)) { ok = false; break; }
    PT_STAMP(3);  // logits received
    uint32_t my_key = 0u;  // wave t < T: the key of top-k position `lane` of token t
    if (wave < T) {  // `red` is free until the work pieces: 64 candidate words per token
      my_key = moe_topk_select<SLOTS>(lg + (size_t)wave * E, E, k, topi + wave * k, (uint64_t*)red + 64 * wave);
      if (MT > 1) moe_topk_weights(my_key, k, topw + wave * k);
    }
    __syncthreads();
    PT_STAMP(4);  // top-k done
    // With one token, unit u < k is top-k choice u and unit k the shared
    // expert: no plan, and the weights are taken once this workgroup's weight
    // loads are in flight (below).  With more tokens: the plan (wave 0).
    auto emit_topk = [&]() {
      if (g == 0 && tid < T * k) {
        if (a.topk_idx_out) a.topk_idx_out[(size_t)l * T * k + tid] = topi[tid];
        if (a.topk_w_out) a.topk_w_out[(size_t)l * T * k + tid] = topw[tid];
      }
    };
    if (MT > 1) {
      emit_topk();
      if (wave == 0)
        pt_plan(topi, T, k, E, lslots, a.record_bytes, true, TS, p_exp, p_ntok, p_tok, p_j, p_roff, p_cum, p_misc,
                (uint32_t*)red, (int*)red + E);  // `red` is free until the work pieces
      __syncthreads();
      PT_STAMP(13);  // plan done
    }
    // ------------------------------------------------------------ work pieces
    // The layer's expert work is cut into pieces of 8 f values: (unit u, piece
    // p) for the units u < U1 of the plan (the shared expert last) and p <
    // F/8.  Piece (u, p) = the gate and up rows of f = 8p..8p+7 over all of K,
    // then those 8 columns of the down matrix.  A group is the 4 pieces of one
    // unit whose down values share a down block column (int4: the 4 words of
    // the 16-byte blocks of column p/4; int2: the two words of blocks p/2), so
    // that one group's gate/up rows are 64 consecutive rows of its record and
    // its down values are 16 bytes (int4) or two words (int2) per row.  With
    // one token, group i = u * F/32 + b (a workgroup's work is one expert's
    // rows); with more, i = b * U1 + u (the units interleaved, so that every
    // workgroup gets the same mix of experts and token counts).  Workgroup g
    // takes the groups [g*NG/G, (g+1)*NG/G) (with single shared pieces: group
    // g and that piece; with more tokens: a range balanced by cost), one
    // batch per group.  In a batch the gate/up rows are split over the 8
    // waves by K and over the lanes as described at load_gu; row slot s
    // (s < 64) of the batch is gate/up row s%16 of piece s/16, slots 64..79
    // the single shared piece (row slot B); the down rows of thread tid are
    // tid + 512 c.
    {
      const int U1 = MT == 1 ? k + 1 : p_misc[0], NB4 = NP / 4, NG = U1 * NB4;
      const PtMask mk = pt_masks(QFMT);
      const bool ilv = T > 1;  // interleaved group order
      int gi0 = (int)((int64_t)g * NG / G), gi1 = (int)((int64_t)(g + 1) * NG / G);
      if (sepB) {
        gi0 = g;
        gi1 = g + 1;
      }
      if (MT > 1) {
        // balanced by cost: group i = b * U1 + u starts at cost b * Crow +
        // p_cum[u]; workgroup g takes the groups starting in [g C/G, (g+1) C/G)
        const int Crow = p_cum[U1];
        const int64_t C = (int64_t)NB4 * Crow;
        auto first_at = [&](int64_t target) -> int {
          if (target >= C) return NG;
          const int b = (int)(target / Crow), rem = (int)(target - (int64_t)b * Crow);
          const uint64_t m = __ballot(lane < U1 && p_cum[lane < U1 ? lane : 0] >= rem);
          int u = m ? __ffsll((long long)m) - 1 : min(U1, 64);
          if (!m)  // units past the wave's 64 lanes (U1 = 65)
            while (u < U1 && p_cum[u] < rem) ++u;
          return b * U1 + u;
        };
        gi0 = first_at((int64_t)g * C / G);
        gi1 = first_at((int64_t)(g + 1) * C / G);
      }
      PT_MARK(14, gi1 - gi0);  // this workgroup's group count
      constexpr int NRD = 4;  // down rows per thread (H <= 2048)
      float y[NRD][MT];
#pragma unroll
      for (int c = 0; c < NRD; ++c)
#pragma unroll
        for (int t = 0; t < MT; ++t) y[c][t] = 0.f;
      auto unit_of = [&](int gi) { return ilv ? gi % U1 : gi / NB4; };
      auto block_of = [&](int gi) { return ilv ? gi / U1 : gi % NB4; };
      auto rec_of = [&](int u) -> const uint8_t* {  // uniform over the workgroup
        return a.pool + (MT == 1 ? (int64_t)lslots[u < k ? topi[u] : E] * a.record_bytes : p_roff[u]);
      };
      // ---- gate/up loads of group gi (its 64 consecutive rows 64 b + rho),
      // 8 16-byte words q and 4 words sc per lane.  Lane l = (p = l % 16,
      // quarter q = l / 16) holds rows rho = p + 16 j (j < 4) over quarter q of
      // the wave's K range, 64 values (int4: blocks 2q, 2q+1 of the wave's 8;
      // int2: q-unit q of its 4): q[j][0..1] = the two blocks (int4) or the
      // q-unit and its meta unit (int2), sc[j] = the two scales (int4).  Each
      // quarter's activations are read from LDS once per token and used for 4
      // rows (a quarter of the LDS traffic of one row per lane); the quarters
      // are summed with shuffles.
      const int lp = lane & 15;
      const int kuq = min(ku0 + (lq >> 1), NKU - 1);  // K unit of the lane's quarter
      const bool kvq = ku0 + (lq >> 1) < ku1;
      auto load_gu = [&](int gi, uint4 (&q)[4][2], uint32_t (&sc)[4]) {
        const uint8_t* rg = rec_of(unit_of(gi));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t row = (uint32_t)(64 * block_of(gi) + lp + 16 * j);
          if (QFMT == MOE_Q4_B32) {
            const uint32_t kb0 = 4u * (uint32_t)kuq + 2u * (lq & 1);
            sc[j] = *reinterpret_cast<const uint32_t*>(rg + (o_gus + 16u * (uint32_t)kuq * (uint32_t)F + 8u * row + 4u * (lq & 1)));
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
              q[j][bb] = *reinterpret_cast<const uint4*>(rg + (o_guq + 16u * ((kb0 + bb) * 2u * (uint32_t)F + row)));
          } else {
            const uint32_t un = 2u * (uint32_t)kuq + (lq & 1);  // q-unit of 64 values
            sc[j] = 0u;
            q[j][0] = *reinterpret_cast<const uint4*>(rg + (o_guq + 16u * (un * 2u * (uint32_t)F + row)));
            q[j][1] = *reinterpret_cast<const uint4*>(rg + (o_gus + 16u * (un * 2u * (uint32_t)F + row)));
          }
        }
      };
      uint4 gq[4][2];
      uint32_t gs[4];
      if (MT > 1) load_gu(min(gi0, NG - 1), gq, gs);  // clamped: every load is unconditional
      for (int gi = gi0; gi < gi1; ++gi) {
        const bool withS = gi == gi0 && sp >= 0;  // the single shared piece rides along
        const int u = unit_of(gi), bq = block_of(gi);
        const int ntok = MT == 1 ? 1 : p_ntok[u];
        const uint8_t* rec = rec_of(u);
        if (MT == 1) load_gu(gi, gq, gs);
        // ---- down loads of the group: int4: the 16-byte block and its scale;
        // int2: the two block words and their two meta words
        uint4 dq[NRD];
        uint32_t dsc[NRD];
        auto load_down = [&]() {
#pragma unroll
          for (int c = 0; c < NRD; ++c) {
            const uint32_t r = (uint32_t)min(tid + 512 * c, H - 1);
            if (QFMT == MOE_Q4_B32) {
              dq[c] = *reinterpret_cast<const uint4*>(rec + (o_dq + 16u * ((uint32_t)bq * (uint32_t)H + r)));
              dsc[c] = *reinterpret_cast<const uint16_t*>(rec + (o_ds + 2u * ((uint32_t)bq * (uint32_t)H + r)));
            } else {
              const uint32_t b0 = 2u * (uint32_t)bq;
              dq[c].x = *reinterpret_cast<const uint32_t*>(rec + (o_dq + 4u * (b0 * (uint32_t)H + r)));
              dq[c].y = *reinterpret_cast<const uint32_t*>(rec + (o_dq + 4u * ((b0 + 1u) * (uint32_t)H + r)));
              dq[c].z = *reinterpret_cast<const uint32_t*>(rec + (o_ds + 4u * (b0 * (uint32_t)H + r)));
              dq[c].w = *reinterpret_cast<const uint32_t*>(rec + (o_ds + 4u * ((b0 + 1u) * (uint32_t)H + r)));
              dsc[c] = 0u;
            }
          }
        };
        load_down();
        __builtin_amdgcn_sched_barrier(0);  // every load above is issued before any dot product
        if (MT == 1 && gi == gi0 && wave == 0) moe_topk_weights(my_key, k, topw);  // read after the next barrier
        // ---- gate/up partial dots
        auto xp_of = [&](int t) -> const uint8_t* {
          return xprep + (size_t)(MT == 1 ? 0 : p_tok[u * TS + t]) * a.prep_bytes;
        };
        {  // the quarter mapping, one token and one block of x at a time
          const int rho = lp + 16 * lq;
          const int slot = 16 * ((rho & 31) >> 3) + (rho & 7) + 8 * (rho >> 5);
#pragma unroll 1
          for (int t = 0; t < ntok; ++t) {
            const uint8_t* xp = xp_of(t);
            const float2* corr = (const float2*)(xp + 2 * (size_t)H);
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
            if (QFMT == MOE_Q4_B32) {
              const int kb0 = 4 * kuq + 2 * (lq & 1);
#pragma unroll
              for (int bb = 0; bb < 2; ++bb) {
                uint32_t xw[16];  // the prepared x of block kb0 + bb
#pragma unroll
                for (int w4 = 0; w4 < 4; ++w4) {
                  const uint4 v = *reinterpret_cast<const uint4*>((const uint32_t*)xp + 16 * (kb0 + bb) + 4 * w4);
                  xw[4 * w4] = v.x; xw[4 * w4 + 1] = v.y; xw[4 * w4 + 2] = v.z; xw[4 * w4 + 3] = v.w;
                }
                const float cb = corr[kb0 + bb].x;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  const float sj = kvq ? moe_f16_to_f32((uint16_t)(gs[j] >> (16 * bb))) : 0.f;
                  acc[j] = fmaf(sj, pt_q4_dot(gq[j][bb], xw, cb, mk), acc[j]);
                }
              }
            } else {
              const int un = 2 * kuq + (lq & 1);
#pragma unroll 2
              for (int jb = 0; jb < 4; ++jb) {
                uint32_t xw[8];  // the prepared x of block 4 un + jb
#pragma unroll
                for (int w4 = 0; w4 < 2; ++w4) {
                  const uint4 v = *reinterpret_cast<const uint4*>((const uint32_t*)xp + 32 * un + 8 * jb + 4 * w4);
                  xw[4 * w4] = v.x; xw[4 * w4 + 1] = v.y; xw[4 * w4 + 2] = v.z; xw[4 * w4 + 3] = v.w;
                }
                const float2 cb = corr[4 * un + jb];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  const uint32_t qw = jb == 0 ? gq[j][0].x : jb == 1 ? gq[j][0].y : jb == 2 ? gq[j][0].z : gq[j][0].w;
                  const uint32_t mw = jb == 0 ? gq[j][1].x : jb == 1 ? gq[j][1].y : jb == 2 ? gq[j][1].z : gq[j][1].w;
                  const float sc = kvq ? moe_f16_to_f32((uint16_t)(mw & 0xffff)) : 0.f;
                  const float mn = kvq ? moe_f16_to_f32((uint16_t)(mw >> 16)) : 0.f;
                  acc[j] += pt_q2_dot(qw, sc, mn, xw, cb, mk);
                }
              }
            }
            // sum over the quarters (lanes l, l ^ 16, l ^ 32, l ^ 48)
            float mine = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              float v = acc[j];
              v += __shfl_xor(v, 16, 64);
              v += __shfl_xor(v, 32, 64);
              mine = lq == j ? v : mine;
            }
            red[(wave * PT_SLOTS + slot) * MT + t] = mine;
          }
        }
        if (MT == 1) {  // row slot B: the single shared piece, 4 lane groups summed with shuffles
          float accB = 0.f;
          const uint8_t* xp = xprep;
          if (QFMT == MOE_Q4_B32) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              const int kb = 4 * kuB + 2 * (lq & 1) + b;
              const float sc = kvB ? moe_f16_to_f32((uint16_t)(gsS >> (16 * b))) : 0.f;
              const float cc = ((const float2*)(xp + 2 * (size_t)H))[kb].x;
              accB = fmaf(sc, pt_q4_dot(gqS[b], (const uint32_t*)xp + 16 * kb, cc, mk), accB);
            }
          } else {
            const uint32_t qw[4] = {gqS[0].x, gqS[0].y, gqS[0].z, gqS[0].w};
            const uint32_t mw[4] = {gqS[1].x, gqS[1].y, gqS[1].z, gqS[1].w};
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
              const int bl = 4 * (2 * kuB + (lq & 1)) + jb;
              const float sc = kvB ? moe_f16_to_f32((uint16_t)(mw[jb] & 0xffff)) : 0.f;
              const float mn = kvB ? moe_f16_to_f32((uint16_t)(mw[jb] >> 16)) : 0.f;
              const float2 cc = ((const float2*)(xp + 2 * (size_t)H))[bl];
              accB += pt_q2_dot(qw[jb], sc, mn, (const uint32_t*)xp + 8 * bl, cc, mk);
            }
          }
          accB += __shfl_xor(accB, 16, 64);
          accB += __shfl_xor(accB, 32, 64);
          red[(wave * PT_SLOTS + 64 + (lane & 15)) * MT] = accB;  // the 4 lane groups hold the same sum
        }
        // several tokens: the next group's gate/up rows are requested now (after
        // this group's down words, so that the down dots need not wait for
        // them) and land while this group's SiLU and down dots run
        uint4 gqN[4][2];
        uint32_t gsN[4];
        if (MT > 1) load_gu(min(gi + 1, gi1 - 1), gqN, gsN);
        __syncthreads();
        PT_STAMP(5);  // gate/up dots done
        if (gi == gi0 + 1) PT_STAMP(12);  // (second group)
        // ---- h = silu(gate) * up, 8 threads per (piece, token slot), then the
        // prepared word of the 8 h values for the down dots
        {
          const int item = tid >> 3, fi = tid & 7;  // item = pi * MT + t
          const int pi = item / MT, t = item % MT;
          const bool iv = pi < 4 || (pi == 4 && withS);
          float hv = 0.f;
          if (iv) {
            float sg = 0.f, su = 0.f;
#pragma unroll
            for (int w = 0; w < PT_WAVES; ++w) {
              sg += red[(w * PT_SLOTS + 16 * pi + fi) * MT + t];
              su += red[(w * PT_SLOTS + 16 * pi + 8 + fi) * MT + t];
            }
            hv = moe_silu(sg) * su;
          }
          const float hn = pt_xor1(hv);  // partner value of the pair
          const int pk = fi >> 1;                   // pair index within the word
          float c0 = 0.f, c1 = 0.f;
          uint32_t pw = 0u;
          if ((fi & 1) == 0) {
            if (QFMT == MOE_Q4_B32) {
              const float mul = (pk & 1) ? 0.0625f : 1.f;
              const half2v a2 = {(_Float16)(hv * mul), (_Float16)(hn * mul)};
              const half2v kk = {(_Float16)((pk & 1) ? 1152.f : 1032.f), (_Float16)((pk & 1) ? 1152.f : 1032.f)};
              pw = moe_half2_as_u32(a2);
              c0 = moe_dot2(a2, kk, 0.f);
            } else {
              const float mul = pk == 0 ? 1.f : pk == 1 ? 0.25f : pk == 2 ? 0.0625f : 0.015625f;
              const half2v a2 = {(_Float16)(hv * mul), (_Float16)(hn * mul)};
              const half2v k1024 = {(_Float16)1024.f, (_Float16)1024.f};
              const half2v kc = {(_Float16)(1.f / mul), (_Float16)(1.f / mul)};
              pw = moe_half2_as_u32(a2);
              c0 = moe_dot2(a2, k1024, 0.f);
              c1 = moe_dot2(a2, kc, 0.f);
            }
          }
          // corrections summed over the 4 pairs (lanes fi = 0, 2, 4, 6 of the
          // item; the sum is complete in lane fi = 0, the one that stores it)
          c0 += pt_xor2(c0);
          c0 += pt_next4(c0);
          c1 += pt_xor2(c1);
          c1 += pt_next4(c1);
          if (iv && item < PT_PB_MAX * MT) {
            if ((fi & 1) == 0) hp[item * 4 + pk] = pw;
            if (fi == 0) hc[item] = make_float2(c0, c1);
          }
        }
        __syncthreads();
        PT_STAMP(6);  // SiLU done
        // ---- down dots: rows tid + 512 c, the group's 4 pieces.  Per window
        // token tt (a register index of y) the unit's entry lt for it, if any
        // (uniform over the workgroup), so that each product is added to one
        // accumulator without selecting among the token slots.
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) {
          int lt = MT == 1 ? 0 : -1;
          if (MT > 1 && tt < T)
            for (int t = 0; t < ntok; ++t)
              if (p_tok[u * TS + t] == tt) lt = t;
          lt = __builtin_amdgcn_readfirstlane(lt);
          if (lt < 0) continue;
          const int jj = MT == 1 ? u : p_j[u * TS + lt];
          const float wgt = jj < k ? topw[tt * k + jj] : 1.f;
#pragma unroll
          for (int pi = 0; pi < 4; ++pi) {
            const uint32_t* hw4 = hp + (pi * MT + lt) * 4;
            const float2 cc = hc[pi * MT + lt];
#pragma unroll
            for (int c = 0; c < NRD; ++c) {
              float v;
              if (QFMT == MOE_Q4_B32) {
                const uint32_t w = pi == 0 ? dq[c].x : pi == 1 ? dq[c].y : pi == 2 ? dq[c].z : dq[c].w;
                v = moe_f16_to_f32((uint16_t)dsc[c]) * pt_q4_word(w, hw4, cc.x, mk);
              } else {
                const uint32_t w = (pi < 2 ? dq[c].x : dq[c].y) >> (8 * (pi & 1));
                const uint32_t m = pi < 2 ? dq[c].z : dq[c].w;
                v = pt_q2_word(w, moe_f16_to_f32((uint16_t)(m & 0xffff)), moe_f16_to_f32((uint16_t)(m >> 16)), hw4, cc, mk);
              }
              y[c][tt] = fmaf(wgt, v, y[c][tt]);
            }
          }
        }
        if (MT == 1 && withS) {  // the single shared piece: weight 1
          const uint32_t* hw4 = hp + 4 * 4;
          const float2 cc = hc[4];
#pragma unroll
          for (int c = 0; c < NRD; ++c) {
            float v;
            if (QFMT == MOE_Q4_B32) {
              v = moe_f16_to_f32((uint16_t)dmS[c]) * pt_q4_word(dwS[c], hw4, cc.x, mk);
            } else {
              const uint32_t w = dwS[c] >> (8 * (sp & 1));
              v = pt_q2_word(w, moe_f16_to_f32((uint16_t)(dmS[c] & 0xffff)), moe_f16_to_f32((uint16_t)(dmS[c] >> 16)),
                             hw4, cc, mk);
            }
            y[c][0] += v;
          }
        }
        __syncthreads();  // red, hp, hc are reused by the next batch
        PT_STAMP(7);  // group done
        if (gi == gi0) PT_STAMP(15);  // first group done
        if (MT > 1) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            gs[j] = gsN[j];
            gq[j][0] = gqN[j][0];
            gq[j][1] = gqN[j][1];
          }
        }
      }
      if (MT == 1) {
        if (gi0 == gi1 && wave == 0) moe_topk_weights(my_key, k, topw);
        emit_topk();  // topw was written before a barrier above (or by this thread's wave, lanes < k)
      }
      // this workgroup's partial output, one vector per token (the thread
      // index is made opaque here so that the compiler computes the NRD * MT
      // offsets now instead of keeping them live across the layer loop)
      int tid_o = tid;
      asm volatile("" : "+v"(tid_o));
#pragma unroll
      for (int c = 0; c < NRD; ++c) {
        const int r = tid_o + 512 * c;
        if (r < H) {
#pragma unroll
          for (int t = 0; t < MT; ++t)
            if (t < T) pt_put(pt_at(a.pbuf, (uint32_t)((g * T + t) * H + r)), tag, y[c][t]);
        }
      }
    }
    // ------------------------------------------------------------ phase C
    {
      // outputs (t, r) for r in this workgroup's rows; TPO threads per output,
      // thread `sub` summing the partials of workgroups sub, sub + TPO, ... in
      // order, then the sum over the TPO lanes (pt_segment_sum, complete in the
      // last of them; a fixed order for a given T)
      const int r0 = g * a.rpw;
      const int nout = T * a.rpw;
      const int tpo = a.tpo;
      constexpr int NQ = MT == 1 ? 8 : MT == 2 ? 12 : MT <= 4 ? 24 : 32;
      // each thread polls its NQ partial words until they all carry the tag
      // (no workgroup barrier per round, no per-producer sentinel pass),
      // then sums them in a fixed order
      for (int ob = 0; ob < nout; ob += PT_THREADS / tpo) {
        const int oo = ob + tid / tpo, sub = tid % tpo;
        const bool act = oo < nout;
        const int t = act ? oo / a.rpw : 0, rr = act ? r0 + oo % a.rpw : r0;
        float sum = 0.f;
        for (int p0 = sub; p0 < G && ok; p0 += tpo * NQ) {
          u64 w[NQ];
          bool need[NQ];  // (one token: reload only the missing words)
#pragma unroll
          for (int qq = 0; qq < NQ; ++qq) need[qq] = act && p0 + tpo * qq < G;
          for (int it = 0;; ++it) {
            bool mine = true;
#pragma unroll
            for (int qq = 0; qq < NQ; ++qq)
              if (MT > 1 || need[qq]) w[qq] = pt_load(a.pbuf, (uint32_t)((min(p0 + tpo * qq, G - 1) * T + t) * H + rr));
#pragma unroll
            for (int qq = 0; qq < NQ; ++qq) {
              if (MT == 1) need[qq] = need[qq] && (uint32_t)(w[qq] >> 32) != tag;
              mine &= !(act && p0 + tpo * qq < G) || (uint32_t)(w[qq] >> 32) == tag;
            }
            if (mine) break;
            if (it > PT_SPIN_MAX) { ok = false; break; }
          }
#pragma unroll
          for (int qq = 0; qq < NQ; ++qq)
            if (act && p0 + tpo * qq < G) sum += __uint_as_float((uint32_t)w[qq]);
        }
        if (!__syncthreads_and(ok)) { ok = false; break; }
        PT_STAMP(8);  // partial sums received
        sum = pt_segment_sum(sum, tpo);
        if (act && sub == tpo - 1) {
          const float xn = xs[t * H + rr] + sum;
          if (l + 1 < L) {
#pragma unroll
            for (int rep = 0; rep < PT_REPL; ++rep)  // one copy per XCD
              pt_put(pt_at(a.xbuf, (uint32_t)((rep * T + t) * H + rr)), tag, xn);
          } else {
            a.x_out[(size_t)t * H + rr] = xn;
          }
        }
      }
      if (!ok) break;
    }
    __syncthreads();
    PT_STAMP(9);  // layer done
  }
  PT_STAMP_FLUSH();
  if (!ok) {
    // the error word: the next call's set-up kernel then zeroes the tagged
    // buffers (this call's tags stay reserved, so this is belt and braces)
    if (tid == 0) __hip_atomic_store(a.hdr + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = g * PT_THREADS + tid; i < T * H; i += G * PT_THREADS) a.x_out[i] = __builtin_nanf("");
    return;
  }
}

// Address of the kernel instance for (qfmt, mt token slots, SLOTS), or NULL.
// The instances are compiled in separate translation units, so that the build
// compiles them in parallel: mt 1 and 2, mt 3 and 4, mt 6 and 8.
const void* pt_kernel_mt12(int qfmt, int mt, int slots);
const void* pt_kernel_mt34(int qfmt, int mt, int slots);
const void* pt_kernel_mt68(int qfmt, int mt, int slots);
#define PT_PICK(Q, M, S) \
  if (qfmt == Q && mt == M && slots == S) return (const void*)decode_persistent_kernel<Q, M, S>;
#define PT_PICK_S(Q, M) PT_PICK(Q, M, 1) PT_PICK(Q, M, 2) PT_PICK(Q, M, 4) PT_PICK(Q, M, 8) PT_PICK(Q, M, 16)
#define PT_PICK_M(M) PT_PICK_S(MOE_Q4_B32, M) PT_PICK_S(MOE_Q2_B16, M)
