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
//     the current (call, layer) tag.  No counters, so nothing serialises.
// Per layer l (tag t_l), workgroup g:
//   A  read x_l (tagged, or x_in for l = 0); mean square -> inv rms;
//      router rows e = g (mod G): logits of xn = x * inv, tagged.
//      Prepare xn for the expert dot products (fp16 pairs) in LDS.
//   B  read all logits; top-k + softmax per token (one wave per token); the
//      plan of distinct experts (computed identically by every workgroup).
//      Work units (distinct expert u, f-slice fs of 32): gate/up rows of fs
//      (all of K) -> h = silu(g) * up for the slice -> the slice's column
//      block of the down matrix times h -> a weighted partial output vector
//      of H rows per token, tagged.  A unit reads its gate/up rows and its
//      down block column at once: one weight stream per layer.
//   C  rows r of workgroup g: x_{l+1}[r] = x_l[r] + sum over the token's
//      k+1 experts and all f-slices of the partials, in a fixed order.
// Every workgroup produces router rows in A and output rows in C, so no
// workgroup can fall a layer behind the data it still has to read.
// Every wait is bounded; on timeout the error word is set, x_out is filled
// with NaN and the kernel ends.
#include "moe_common.h"
#include "moe_sizes.h"
#include "moe_kernels.h"

#define PT_THREADS 512
#define PT_WAVES 8
#define PT_SPIN_MAX (1 << 18)
#define PT_MAGIC 0x4d6f4531u
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
  uint32_t* hdr;  // [0] magic, [1] call counter, [2] error
  u64* xbuf;      // [T][H]
  u64* lbuf;      // [T][E]
  u64* pbuf;      // [(unit * T + i)][H]
  int G, nfs, rpw, tpo;
  size_t prep_bytes;
};

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
__device__ __forceinline__ uint32_t pt_tag(uint32_t call, int L, int l) {
  return (uint32_t)(((uint64_t)call * (uint64_t)L + (uint64_t)l) % 0xFFFFFFFFull) + 1u;
}

// ---------------------------------------------------------------- small helpers
// dot of one int4 block (16 bytes) with a prepared activation block
__device__ __forceinline__ float pt_q4_dot(uint4 q, const uint32_t* xp, float c) {
  const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
  float d = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = qw[j], w8 = qw[j] >> 8;
    d = moe_dot2(moe_u32_as_half2((w & 0x000F000Fu) | MOE_F16_1024X2), moe_u32_as_half2(xp[4 * j + 0]), d);
    d = moe_dot2(moe_u32_as_half2((w & 0x00F000F0u) | MOE_F16_1024X2), moe_u32_as_half2(xp[4 * j + 1]), d);
    d = moe_dot2(moe_u32_as_half2((w8 & 0x000F000Fu) | MOE_F16_1024X2), moe_u32_as_half2(xp[4 * j + 2]), d);
    d = moe_dot2(moe_u32_as_half2((w8 & 0x00F000F0u) | MOE_F16_1024X2), moe_u32_as_half2(xp[4 * j + 3]), d);
  }
  return d - c;
}
// one int2 block (one word) with a prepared block: s * (dot - c0) + m * sum(x)
__device__ __forceinline__ float pt_q2_dot(uint32_t w, float s, float m, const uint32_t* xp, float2 c) {
  const uint32_t w8 = w >> 8;
  float d = 0.f;
  d = moe_dot2(moe_u32_as_half2((w & 0x00030003u) | MOE_F16_1024X2), moe_u32_as_half2(xp[0]), d);
  d = moe_dot2(moe_u32_as_half2((w & 0x000C000Cu) | MOE_F16_1024X2), moe_u32_as_half2(xp[1]), d);
  d = moe_dot2(moe_u32_as_half2((w & 0x00300030u) | MOE_F16_1024X2), moe_u32_as_half2(xp[2]), d);
  d = moe_dot2(moe_u32_as_half2((w & 0x00C000C0u) | MOE_F16_1024X2), moe_u32_as_half2(xp[3]), d);
  d = moe_dot2(moe_u32_as_half2((w8 & 0x00030003u) | MOE_F16_1024X2), moe_u32_as_half2(xp[4]), d);
  d = moe_dot2(moe_u32_as_half2((w8 & 0x000C000Cu) | MOE_F16_1024X2), moe_u32_as_half2(xp[5]), d);
  d = moe_dot2(moe_u32_as_half2((w8 & 0x00300030u) | MOE_F16_1024X2), moe_u32_as_half2(xp[6]), d);
  d = moe_dot2(moe_u32_as_half2((w8 & 0x00C000C0u) | MOE_F16_1024X2), moe_u32_as_half2(xp[7]), d);
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

// wave-wide max of uint32 through DPP row operations and row read-out
__device__ __forceinline__ uint32_t pt_wave_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false)); // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false)); // row_mirror
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Top-k of one token's E logits (LDS) by one wave.  Lane l holds the keys of
// experts l + 64 * i (i < SLOTS): the order-preserving logit bits, and on
// equal bits the lower expert first.  Each lane sorts its keys; every round
// takes the wave-wide maximum of the lane heads and the lane holding it pops
// its head.  Lane j < k ends with the j-th expert and its softmax weight over
// the k chosen logits (ids[j], wts[j]).
template <int SLOTS>
__device__ __forceinline__ void pt_topk(const float* lg, int E, int k, int* ids, float* wts) {
  const int lane = threadIdx.x & 63;
  uint32_t hi[SLOTS], ex[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e = lane + 64 * i;
    hi[i] = e < E ? moe_f32_order_key(lg[e < E ? e : 0]) : 0u;  // every real key has hi > 0
    ex[i] = (uint32_t)e;
  }
  // descending sort of the lane's keys (odd-even transposition network); the
  // experts of one lane ascend with i, so equal keys keep the lower expert first
#pragma unroll
  for (int r = 0; r < SLOTS; ++r) {
#pragma unroll
    for (int i = r & 1; i + 1 < SLOTS; i += 2) {
      const bool sw = hi[i] < hi[i + 1] || (hi[i] == hi[i + 1] && ex[i] > ex[i + 1]);
      const uint32_t h0 = hi[i], e0 = ex[i];
      hi[i] = sw ? hi[i + 1] : hi[i];
      ex[i] = sw ? ex[i + 1] : ex[i];
      hi[i + 1] = sw ? h0 : hi[i + 1];
      ex[i + 1] = sw ? e0 : ex[i + 1];
    }
  }
  uint32_t my_key = 0u, my_e = 0u;
  for (int j = 0; j < k; ++j) {
    const uint32_t M = pt_wave_max(hi[0]);
    const uint64_t cand = __ballot(hi[0] == M);
    int wl = __ffsll((long long)cand) - 1;
    if (__popcll(cand) > 1) {  // equal logits in several lanes: the lowest expert
      const uint32_t ce = hi[0] == M ? ex[0] : 0xFFFFFFFFu;
      const uint32_t emin = ~pt_wave_max(~ce);
      wl = (int)(emin & 63);
    }
    const uint32_t ew = __builtin_amdgcn_readlane(ex[0], wl);
    if (lane == j) {
      my_key = M;
      my_e = ew;
    }
    if (lane == wl) {  // pop the head
#pragma unroll
      for (int i = 0; i + 1 < SLOTS; ++i) {
        hi[i] = hi[i + 1];
        ex[i] = ex[i + 1];
      }
      hi[SLOTS - 1] = 0u;
    }
  }
  // softmax over the chosen logits, lane j holding logit j (max is lane 0's)
  const float m0 = moe_order_key_f32(__builtin_amdgcn_readfirstlane(my_key));
  const float z = lane < k ? expf(moe_order_key_f32(my_key) - m0) : 0.f;
  float sum = z;  // sum in lane order: lanes 0..k-1 are added left to right
  {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), j));
    sum = acc;
  }
  if (lane < k) {
    ids[lane] = (int)my_e;
    wts[lane] = z / sum;
  }
}

// Work plan of one layer from the T * k chosen experts (one wave): the
// distinct experts in order of first occurrence (token-major), each with its
// tokens and their top-k positions, then the shared expert with every token.
// uslot[t * (k + 1) + j] = u * 4 + c names the unit u and token slot c that
// produce token t's j-th expert output.  n = T * k <= 64.
__device__ __forceinline__ void pt_plan(const int* topi, int T, int k, int E, int* p_exp, int* p_ntok, int* p_tok,
                                        int* p_j, int* uslot, int* p_misc) {
  const int lane = threadIdx.x & 63, n = T * k;
  const int e = lane < n ? topi[lane] : -1 - lane;  // distinct negatives for idle lanes
  int first = lane, before = 0, total = 0;           // first lane with this expert; count before; count
  for (int q = 0; q < n; ++q) {
    const int eq = __builtin_amdgcn_readlane(e, q);
    if (eq == e) {
      first = min(first, q);
      before += q < lane;
      ++total;
    }
  }
  const uint64_t firsts = __ballot(lane < n && first == lane);
  const int u_first = (int)__popcll(firsts & ((1ull << lane) - 1ull));  // rank among first occurrences
  const int u = __shfl(u_first, first, 64);
  const int U = (int)__popcll(firsts);
  if (lane < n) {
    const int t = lane / k, j = lane % k;
    if (first == lane) {
      p_exp[u] = e;
      p_ntok[u] = total;
    }
    p_tok[u * 4 + before] = t;
    p_j[u * 4 + before] = j;
    uslot[t * (k + 1) + j] = u * 4 + before;
  }
  if (lane < T) {
    p_tok[U * 4 + lane] = lane;
    p_j[U * 4 + lane] = k;
    uslot[lane * (k + 1) + k] = U * 4 + lane;
  }
  if (lane == 0) {
    p_exp[U] = E;
    p_ntok[U] = T;
    p_misc[0] = U + 1;
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
    c0 += __shfl_xor(c0, 1, 64);
    c0 += __shfl_xor(c0, 2, 64);
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
    c0 += __shfl_xor(c0, 1, 64);
    c1 += __shfl_xor(c1, 1, 64);
    if (valid && sub == 0) *corr = make_float2(c0, c1);
  }
}

// ---------------------------------------------------------------- LDS layout
// Section offsets (bytes, 16-byte aligned) shared by the kernel and the host.
// Per-half sections (red, hs, hp, hc) exist twice: the two halves of the
// workgroup run two work units side by side.
struct PtLds {
  size_t xs, xprep, lg, topi, topw, p_exp, p_ntok, p_tok, p_j, p_misc, red, hp, hc, inv, hs, uslot, poff, total;
};
__host__ __device__ inline PtLds pt_lds(int qfmt, int T, int k, int E, int H, int nfs, size_t prep_bytes) {
  PtLds o;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = (off + bytes + 15) / 16 * 16;
    return at;
  };
  const size_t U1max = (size_t)T * k + 1;
  o.xs = take((size_t)T * H * 4);
  o.xprep = take((size_t)T * prep_bytes);
  o.lg = take((size_t)T * E * 4);
  o.topi = take((size_t)T * k * 4);
  o.topw = take((size_t)T * k * 4);
  o.p_exp = take(U1max * 4);
  o.p_ntok = take(U1max * 4);
  o.p_tok = take(U1max * 16);
  o.p_j = take(U1max * 16);
  o.p_misc = take(16);
  o.red = take((size_t)2 * 4 * 4 * 64 * 4);  // [half][wave][token][64]
  o.hp = take(2 * 4 * 16 * 4);                // [half][token][16]
  o.hc = take(2 * 4 * 2 * 8);                 // [half][token][2]
  o.inv = take(4 * 4);
  o.hs = take(2 * 4 * 32 * 4);                // [half][token][32]
  o.uslot = take((size_t)T * (k + 1) * 4);
  o.poff = take((size_t)T * (k + 1) * nfs * 4);
  o.total = off;
  return o;
}

// ---------------------------------------------------------------- the kernel
template <int QFMT, int MT, int SLOTS>
__global__ __launch_bounds__(PT_THREADS) void decode_persistent_kernel(PtArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int T = a.T, H = a.H, F = a.F, E = a.E, k = a.k, L = a.L, G = a.G;
  const int tid = threadIdx.x, lane = tid & 63, g = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave >> 2, hw = wave & 3, htid = tid & 255;  // two 4-wave halves
  const int blk = QFMT == MOE_Q4_B32 ? 32 : 16;
  const MoePlanes pl = moe_planes(QFMT, H, F);  // a record is < 4 GiB: 32-bit plane offsets
  const uint32_t o_guq = (uint32_t)pl.gu_q, o_gus = (uint32_t)pl.gu_s, o_dq = (uint32_t)pl.d_q, o_ds = (uint32_t)pl.d_s;

  const PtLds o = pt_lds(QFMT, T, k, E, H, a.nfs, a.prep_bytes);
  float* xs = (float*)(smem + o.xs);          // [T][H]
  uint8_t* xprep = smem + o.xprep;            // [T][prep_bytes]
  float* lg = (float*)(smem + o.lg);          // [T][E]
  int* topi = (int*)(smem + o.topi);          // [T][k]
  float* topw = (float*)(smem + o.topw);      // [T][k]
  int* p_exp = (int*)(smem + o.p_exp);        // [U1max]
  int* p_ntok = (int*)(smem + o.p_ntok);      // [U1max]
  int* p_tok = (int*)(smem + o.p_tok);        // [U1max][4]
  int* p_j = (int*)(smem + o.p_j);            // [U1max][4]
  int* p_misc = (int*)(smem + o.p_misc);      // [0] = U1
  float* red = (float*)(smem + o.red);        // [2][4][4][64]
  uint32_t* hp = (uint32_t*)(smem + o.hp);    // [2][4][16]
  float2* hc = (float2*)(smem + o.hc);        // [2][4][2]
  float* inv = (float*)(smem + o.inv);        // [4]
  float* hs = (float*)(smem + o.hs);          // [2][4][32]
  int* uslot = (int*)(smem + o.uslot);        // [T][k+1] -> u * 4 + i
  uint32_t* poff = (uint32_t*)(smem + o.poff); // [T][(k+1) * nfs]

  const uint32_t call = __hip_atomic_load(a.hdr + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  bool ok = true;
  const int nrch = (H + 511) / 512;  // router chunks of 512 columns per row (<= 4)
  const int nparts = (k + 1) * a.nfs;  // partial vectors summed into one output row

  for (int l = 0; l < L && ok; ++l) {
    const uint32_t tag = pt_tag(call, L, l);
    // ------------------------------------------------------------ phase A
    // this wave's router row (if any) is requested before waiting for x_l
    // (indices are clamped into range so that every load is unconditional)
    const uint16_t* wr = a.w_router + (size_t)l * E * H;  // wave-uniform; 32-bit offsets below
    const int e_row = g + G * wave;
    uint4 rw[4];
    if (e_row < E) {  // wave-uniform
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t h0 = 512 * c + 8 * lane;
        rw[c] = *reinterpret_cast<const uint4*>(wr + (uint32_t)e_row * (uint32_t)H + (h0 < (uint32_t)H ? h0 : 0u));
      }
    }
    constexpr int NX = 4 * MT;  // words of x per thread: T * H <= 512 * NX
    if (l == 0) {
      for (int i = tid; i < T * H; i += PT_THREADS) xs[i] = a.x_in[i];
    } else {
      const uint32_t ptag = pt_tag(call, L, l - 1);
      const int last = T * H - 1;
      for (int it = 0;; ++it) {
        u64 w[NX];
#pragma unroll
        for (int q = 0; q < NX; ++q) w[q] = pt_load(a.xbuf, (uint32_t)min(tid + q * PT_THREADS, last));
        bool mine = true;
#pragma unroll
        for (int q = 0; q < NX; ++q) mine &= (uint32_t)(w[q] >> 32) == ptag;
        if (__syncthreads_and(mine)) {
#pragma unroll
          for (int q = 0; q < NX; ++q)
            if (tid + q * PT_THREADS <= last) xs[tid + q * PT_THREADS] = __uint_as_float((uint32_t)w[q]);
          break;
        }
        if (it > PT_SPIN_MAX) { ok = false; break; }
        __builtin_amdgcn_s_sleep(2);
      }
      if (!ok) break;
    }
    __syncthreads();
    // mean square of token t by wave t: lane sums in column order, then the wave
    if (wave < T) {
      float ss = 0.f;
      for (int h = lane; h < H; h += 64) ss = fmaf(xs[wave * H + h], xs[wave * H + h], ss);
      ss = moe_wave_sum(ss);
      if (lane == 0) inv[wave] = 1.0f / sqrtf(ss / (float)H + PT_EPS);
    }
    if (a.x_hist && g == 0)
      for (int i = tid; i < T * H; i += PT_THREADS) a.x_hist[(size_t)l * T * H + i] = xs[i];
    __syncthreads();
    // router rows: the prefetched one, then any further rows of this wave
    for (int e = e_row; e < E; e += G * PT_WAVES) {
      if (e != e_row) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t h0 = 512 * c + 8 * lane;
          rw[c] = *reinterpret_cast<const uint4*>(wr + (uint32_t)e * (uint32_t)H + (h0 < (uint32_t)H ? h0 : 0u));
        }
      }
      float acc[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int h0 = 512 * c + 8 * lane;
        if (c < nrch && h0 < H) {
          const uint32_t ww[4] = {rw[c].x, rw[c].y, rw[c].z, rw[c].w};
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            if (t < T) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {  // the 4 words (8 bf16) of the chunk
                acc[t] = fmaf(xs[t * H + h0 + 2 * i], __uint_as_float(ww[i] << 16), acc[t]);
                acc[t] = fmaf(xs[t * H + h0 + 2 * i + 1], __uint_as_float(ww[i] & 0xffff0000u), acc[t]);
              }
            }
          }
        }
      }
      const float b = a.bias ? a.bias[(size_t)l * E + e] : 0.f;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if (t < T) {
          const float s = moe_wave_sum(acc[t]);
          if (lane == t) pt_put(pt_at(a.lbuf, (uint32_t)(t * E + e)), tag, s * inv[t] + b);
        }
      }
    }
    // prepared xn for the gate/up dot products: one 8-value word per thread
    {
      const int nwords = T * H / 8;
      for (int w0 = 0; w0 < nwords; w0 += PT_THREADS) {
        const int wi = w0 + tid;
        const bool valid = wi < nwords;
        const int t = valid ? wi / (H / 8) : 0, wh = valid ? wi % (H / 8) : 0;  // word within the token
        const int b = wh / (blk / 8), sub = wh % (blk / 8);
        uint8_t* out = xprep + (size_t)t * a.prep_bytes;
        pt_prep_word<QFMT>(xs + (size_t)t * H + 8 * wh, inv[t], valid, (uint32_t*)out + (blk / 2) * b + 4 * sub,
                           (float2*)(out + 2 * (size_t)H) + b, sub);
      }
    }
    // ------------------------------------------------------------ phase B
    for (int it = 0;; ++it) {
      constexpr int NLG = MT * SLOTS / 8 > 0 ? MT * SLOTS / 8 : 1;  // T * E <= 512 * NLG
      const int last = T * E - 1;
      u64 w[NLG];
#pragma unroll
      for (int q = 0; q < NLG; ++q) w[q] = pt_load(a.lbuf, (uint32_t)min(tid + q * PT_THREADS, last));
      bool mine = true;
#pragma unroll
      for (int q = 0; q < NLG; ++q) mine &= (uint32_t)(w[q] >> 32) == tag;
      if (__syncthreads_and(mine)) {
#pragma unroll
        for (int q = 0; q < NLG; ++q)
          if (tid + q * PT_THREADS <= last) lg[tid + q * PT_THREADS] = __uint_as_float((uint32_t)w[q]);
        break;
      }
      if (it > PT_SPIN_MAX) { ok = false; break; }
      __builtin_amdgcn_s_sleep(2);
    }
    if (!ok) break;
    __syncthreads();
    if (wave < T) pt_topk<SLOTS>(lg + (size_t)wave * E, E, k, topi + wave * k, topw + wave * k);
    __syncthreads();
    if (g == 0 && tid < T * k) {
      if (a.topk_idx_out) a.topk_idx_out[(size_t)l * T * k + tid] = topi[tid];
      if (a.topk_w_out) a.topk_w_out[(size_t)l * T * k + tid] = topw[tid];
    }
    // plan (wave 0), then the partial-offset table
    {
      if (wave == 0) pt_plan(topi, T, k, E, p_exp, p_ntok, p_tok, p_j, uslot, p_misc);
      __syncthreads();
      // word offset in pbuf (without the row) of partial pi = j * nfs + fs of
      // token t: unit v = u * nfs + fs, token slot i, both from uslot
      for (int q = tid; q < T * nparts; q += PT_THREADS) {
        const int t = q / nparts, pi = q % nparts, j = pi / a.nfs, fs = pi % a.nfs;
        const int us = uslot[t * (k + 1) + j];
        poff[q] = (uint32_t)((((us >> 2) * a.nfs + fs) * T + (us & 3)) * H);
      }
      __syncthreads();
    }
    const int nunits = p_misc[0] * a.nfs;
    // work units: half h of workgroup g takes unit base + h * G + g
    float* hred = red + half * 4 * 4 * 64;
    float* hhs = hs + half * 4 * 32;
    uint32_t* hhp = hp + half * 4 * 16;
    float2* hhc = hc + half * 4 * 2;
    for (int base = 0; base < nunits; base += 2 * G) {
      const int v = base + half * G + g;
      const bool act = v < nunits;
      const int u = act ? v / a.nfs : 0, fs = act ? v % a.nfs : 0;
      const int ntok = __builtin_amdgcn_readfirstlane(act ? p_ntok[u] : 0);
      const int e = __builtin_amdgcn_readfirstlane(p_exp[u]);
      const int slot = __builtin_amdgcn_readfirstlane(a.slot_table[(size_t)l * (E + 1) + e]);
      const uint8_t* rec = a.pool + (int64_t)slot * a.record_bytes;  // wave-uniform base; 32-bit offsets below
      const uint8_t* xpt[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) xpt[i] = xprep + (size_t)p_tok[u * 4 + (i < ntok ? i : 0)] * a.prep_bytes;
      float acc[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) acc[i] = 0.f;
      // the down block column: thread htid holds rows htid + 256 * c (the
      // rows it multiplies later).  With one token per unit the loads are
      // issued right after the gate/up loads (which are needed first); with
      // more tokens after the gate/up dot products, to bound live registers.
      // A fixed count of 8 rows (H <= 2048); rows past H repeat the last row.
      constexpr bool down_early = MT == 1;
      uint4 dq[8];     // int4: the row's block; int2: two words, two metas
      uint32_t ds[8];  // int4: the row's scale
      auto issue_down = [&]() {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint32_t rr = (uint32_t)(htid + 256 * min(c, H / 256 - 1));
          if (QFMT == MOE_Q4_B32) {
            dq[c] = *reinterpret_cast<const uint4*>(rec + (o_dq + 16u * ((uint32_t)fs * (uint32_t)H + rr)));
            ds[c] = *reinterpret_cast<const uint16_t*>(rec + (o_ds + 2u * ((uint32_t)fs * (uint32_t)H + rr)));
          } else {
            const uint32_t w0 = (2u * fs) * (uint32_t)H + rr, w1 = w0 + (uint32_t)H;
            dq[c].x = *reinterpret_cast<const uint32_t*>(rec + (o_dq + 4u * w0));
            dq[c].y = *reinterpret_cast<const uint32_t*>(rec + (o_dq + 4u * w1));
            dq[c].z = *reinterpret_cast<const uint32_t*>(rec + (o_ds + 4u * w0));
            dq[c].w = *reinterpret_cast<const uint32_t*>(rec + (o_ds + 4u * w1));
          }
        }
      };
      if (act) {
        const int r = 64 * fs + lane;  // gate/up row
        // wave hw takes a quarter of the K blocks, in groups of 4 blocks (the
        // unit of the scale planes); indices are clamped so that every load
        // is unconditional and all of them are in flight together
        if (QFMT == MOE_Q4_B32) {
          const int NG = H / 128, g0 = hw * NG / 4, g1 = (hw + 1) * NG / 4;  // <= 4 groups
          uint4 q[16];
          uint2 sc[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t gg = (uint32_t)min(g0 + c, NG - 1);
            sc[c] = *reinterpret_cast<const uint2*>(rec + (o_gus + 16u * (gg * (uint32_t)F) + 8u * (uint32_t)r));
#pragma unroll
            for (int b = 0; b < 4; ++b)
              q[4 * c + b] = *reinterpret_cast<const uint4*>(rec + (o_guq + 16u * ((4u * gg + b) * 2u * (uint32_t)F + (uint32_t)r)));
          }
          if (down_early) issue_down();
          // with one token every use is unconditional (a group past g1 gets
          // scale 0), so the loads stay together ahead of the first dot
          // product and the down loads behind them stay in flight
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int gg = min(g0 + c, NG - 1);
            const bool gv = g0 + c < g1;
            if (MT > 1 && !gv) continue;
            const uint32_t sw[2] = {sc[c].x, sc[c].y};
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const int kb = 4 * gg + b;
              const float s = gv ? moe_f16_to_f32((uint16_t)(sw[b >> 1] >> (16 * (b & 1)))) : 0.f;
#pragma unroll
              for (int i = 0; i < MT; ++i) {
                if ((MT == 1 && i == 0) || i < ntok) {
                  const float cc = ((const float2*)(xpt[i] + 2 * (size_t)H))[kb].x;
                  acc[i] = fmaf(s, pt_q4_dot(q[4 * c + b], (const uint32_t*)xpt[i] + 16 * kb, cc), acc[i]);
                }
              }
            }
          }
        } else {
          const int U4 = H / 64, u0 = hw * U4 / 4, u1 = (hw + 1) * U4 / 4;  // <= 8 units
          uint4 q[8], m[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const uint32_t uu = (uint32_t)min(u0 + c, U4 - 1);
            q[c] = *reinterpret_cast<const uint4*>(rec + (o_guq + 16u * (uu * 2u * (uint32_t)F + (uint32_t)r)));
            m[c] = *reinterpret_cast<const uint4*>(rec + (o_gus + 16u * (uu * 2u * (uint32_t)F + (uint32_t)r)));
          }
          if (down_early) issue_down();
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const int uu = min(u0 + c, U4 - 1);
            const bool uv = u0 + c < u1;  // past u1: scale and min 0
            if (MT > 1 && !uv) continue;
            const uint32_t qw[4] = {q[c].x, q[c].y, q[c].z, q[c].w}, mw[4] = {m[c].x, m[c].y, m[c].z, m[c].w};
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
              const int b = 4 * uu + jb;
              const float s = uv ? moe_f16_to_f32((uint16_t)(mw[jb] & 0xffff)) : 0.f;
              const float mm = uv ? moe_f16_to_f32((uint16_t)(mw[jb] >> 16)) : 0.f;
#pragma unroll
              for (int i = 0; i < MT; ++i) {
                if ((MT == 1 && i == 0) || i < ntok) {
                  const float2 cc = ((const float2*)(xpt[i] + 2 * (size_t)H))[b];
                  acc[i] += pt_q2_dot(qw[jb], s, mm, (const uint32_t*)xpt[i] + 8 * b, cc);
                }
              }
            }
          }
        }
      }
      if (!down_early && act) issue_down();
#pragma unroll
      for (int i = 0; i < MT; ++i) hred[(hw * 4 + i) * 64 + lane] = acc[i];
      __syncthreads();
      if (act && hw == 0) {
        for (int i = 0; i < ntok; ++i) {
          const float sg = ((hred[(0 * 4 + i) * 64 + lane] + hred[(1 * 4 + i) * 64 + lane]) +
                            hred[(2 * 4 + i) * 64 + lane]) + hred[(3 * 4 + i) * 64 + lane];
          const float up = __shfl(sg, (lane + 32) & 63, 64);
          if (lane < 32) hhs[i * 32 + lane] = moe_silu(sg) * up;
        }
      }
      __syncthreads();
      if (act && htid < ntok * (QFMT == MOE_Q4_B32 ? 1 : 2)) {
        const int i = QFMT == MOE_Q4_B32 ? htid : htid >> 1, b = QFMT == MOE_Q4_B32 ? 0 : htid & 1;
        pt_prep_block<QFMT>(hhs + i * 32 + 16 * b, 1.0f, hhp + i * 16 + 8 * b, hhc + i * 2 + b);
      }
      __syncthreads();
      if (act) {
        float wgt[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          wgt[i] = 1.f;
          if (i < ntok) {
            const int t = p_tok[u * 4 + i], j = p_j[u * 4 + i];
            if (j < k) wgt[i] = topw[t * k + j];
          }
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          if (c >= H / 256) break;
          const int rr = htid + 256 * c;
          float y[MT];
#pragma unroll
          for (int i = 0; i < MT; ++i) y[i] = 0.f;
          if (QFMT == MOE_Q4_B32) {
            const float s = moe_f16_to_f32((uint16_t)ds[c]);
#pragma unroll
            for (int i = 0; i < MT; ++i)
              if (i < ntok) y[i] = s * pt_q4_dot(dq[c], hhp + i * 16, hhc[i * 2].x);
          } else {
            const uint32_t wv[2] = {dq[c].x, dq[c].y}, mv[2] = {dq[c].z, dq[c].w};
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              const float s = moe_f16_to_f32((uint16_t)(mv[b] & 0xffff)), mm = moe_f16_to_f32((uint16_t)(mv[b] >> 16));
#pragma unroll
              for (int i = 0; i < MT; ++i)
                if (i < ntok) y[i] += pt_q2_dot(wv[b], s, mm, hhp + i * 16 + 8 * b, hhc[i * 2 + b]);
            }
          }
#pragma unroll
          for (int i = 0; i < MT; ++i)
            if (i < ntok) pt_put(pt_at(a.pbuf, (uint32_t)((v * T + i) * H + rr)), tag, y[i] * wgt[i]);
        }
      }
      __syncthreads();
    }
    // ------------------------------------------------------------ phase C
    {
      // outputs (t, r) for r in this workgroup's rows; TPO threads per output,
      // thread `sub` summing partials sub, sub + TPO, ... in order, then a
      // butterfly over the TPO lanes (a fixed order for a given T)
      const int r0 = g * a.rpw;
      const int nout = T * a.rpw;
      const int tpo = a.tpo;
      constexpr int NQ = MT == 1 ? 8 : MT == 2 ? 12 : 24;
      for (int ob = 0; ob < nout && ok; ob += PT_THREADS / tpo) {
        const int oo = ob + tid / tpo, sub = tid % tpo;
        const bool act = oo < nout;
        const int t = act ? oo / a.rpw : 0, rr = act ? r0 + oo % a.rpw : r0;
        const uint32_t* po = poff + t * nparts;
        float sum = 0.f;
        for (int it = 0;; ++it) {
          bool mine = true;
          float sacc = 0.f;
          for (int p0 = sub; p0 < nparts; p0 += tpo * NQ) {
            u64 w[NQ];
#pragma unroll
            for (int q = 0; q < NQ; ++q) w[q] = pt_load(a.pbuf, po[min(p0 + tpo * q, nparts - 1)] + (uint32_t)rr);
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
              if (p0 + tpo * q < nparts) {
                if ((uint32_t)(w[q] >> 32) == tag) sacc += __uint_as_float((uint32_t)w[q]);
                else mine = false;
              }
            }
          }
          sum = sacc;
          if (__syncthreads_and(mine || !act)) break;
          if (it > PT_SPIN_MAX) { ok = false; break; }
          __builtin_amdgcn_s_sleep(2);
        }
        if (!ok) break;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1)
          if (m < tpo) sum += __shfl_xor(sum, m, 64);
        if (act && sub == 0) {
          const float xn = xs[t * H + rr] + sum;
          if (l + 1 < L) pt_put(pt_at(a.xbuf, (uint32_t)(t * H + rr)), tag, xn);
          else a.x_out[(size_t)t * H + rr] = xn;
        }
      }
      if (!ok) break;
    }
    __syncthreads();
  }
  if (!ok) {
    if (tid == 0) __hip_atomic_store(a.hdr + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = g * PT_THREADS + tid; i < T * H; i += G * PT_THREADS) a.x_out[i] = __builtin_nanf("");
    return;
  }
  if (g == 0 && tid == 0) __hip_atomic_store(a.hdr + 1, call + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Zeroes the tagged buffers once per workspace (recognised by a magic word).
__global__ void decode_persistent_init_kernel(uint32_t* hdr, u64* buf, size_t nwords) {
  if (hdr[0] == PT_MAGIC) return;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += (size_t)gridDim.x * blockDim.x)
    buf[i] = 0ull;
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    hdr[1] = 0;
    hdr[2] = 0;
  }
}
__global__ void decode_persistent_mark_kernel(uint32_t* hdr) {
  if (threadIdx.x == 0) hdr[0] = PT_MAGIC;
}

// ---------------------------------------------------------------- host side
struct PtLayout {
  size_t hdr, xbuf, lbuf, pbuf, total;
  int G, nfs, rpw;
  size_t prep_bytes, lds;
};

static int pt_grid(int H, int E) {
  static int ncu = 0;
  if (!ncu) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      ncu = 0;
    if (ncu <= 0) ncu = 256;
  }
  int lim = ncu < E ? ncu : E;
  if (H / 8 < lim) lim = H / 8;
  int G = 1;
  while (G * 2 <= lim && H % (G * 2) == 0) G *= 2;
  return G;
}

static PtLayout pt_layout(int T, int k, int E, int H, int F, int qfmt, int G) {
  PtLayout P;
  P.G = G;
  P.nfs = F / 32;
  P.rpw = H / G;
  P.prep_bytes = moe_prep_bytes(H, qfmt);
  const int U1max = T * k + 1;
  P.hdr = 0;
  P.xbuf = 256;
  P.lbuf = P.xbuf + moe_ws_up((size_t)T * H * 8);
  P.pbuf = P.lbuf + moe_ws_up((size_t)T * E * 8);
  P.total = P.pbuf + moe_ws_up((size_t)U1max * P.nfs * T * H * 8);
  P.lds = pt_lds(qfmt, T, k, E, H, P.nfs, P.prep_bytes).total;
  return P;
}

size_t moe_ws_stack_persistent(int T, int k, int E, int H, int F, int qfmt) {
  return pt_layout(T, k, E, H, F, qfmt, 1).total;  // independent of G
}

// LDS one workgroup may reserve (the device's opt-in limit; 64 KB if unknown)
static size_t pt_lds_limit() {
  static size_t lim = 0;
  if (!lim) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeSharedMemPerBlockOptin, dev) == hipSuccess && v > 0)
      lim = (size_t)v;
    else
      lim = 64 * 1024;
  }
  return lim;
}

bool moe_persistent_supported(int T, int k, int E, int H, int F, int qfmt) {
  if (T < 1 || T > 4 || k > MOE_MAX_K) return false;
  const PtLayout P = pt_layout(T, k, E, H, F, qfmt, 1);
  // x words per thread (T * H / 512) and router chunks (H / 512) are unrolled
  // up to 4 * MT and 4: H <= 2048
  return P.lds <= pt_lds_limit() && H <= 2048 && H % 256 == 0;
}

int moe_launch_decode_persistent(const float* x_in, int T, int H, int F, int E, int k, int L,
                                 const uint16_t* w_router, const float* bias, const int32_t* slot_table,
                                 const void* pool, int64_t record_bytes, int qfmt, float* x_out,
                                 int32_t* topk_idx_out, float* topk_w_out, float* x_hist, void* ws,
                                 hipStream_t st) {
  const int G = pt_grid(H, E);
  const PtLayout P = pt_layout(T, k, E, H, F, qfmt, G);
  uint8_t* w = (uint8_t*)ws;
  PtArgs a;
  a.x_in = x_in; a.T = T; a.H = H; a.F = F; a.E = E; a.k = k; a.L = L; a.qfmt = qfmt;
  a.w_router = w_router; a.bias = bias; a.slot_table = slot_table; a.pool = (const uint8_t*)pool;
  a.record_bytes = record_bytes; a.x_out = x_out; a.topk_idx_out = topk_idx_out; a.topk_w_out = topk_w_out;
  a.x_hist = x_hist; a.hdr = (uint32_t*)(w + P.hdr); a.xbuf = (u64*)(w + P.xbuf); a.lbuf = (u64*)(w + P.lbuf);
  a.pbuf = (u64*)(w + P.pbuf); a.G = G; a.nfs = P.nfs; a.rpw = P.rpw; a.prep_bytes = P.prep_bytes;
  {  // threads per output row in the final sum: a power of two <= 64
    int tpo = 64;
    while (tpo > 1 && (size_t)T * P.rpw * tpo > PT_THREADS) tpo >>= 1;
    a.tpo = tpo;
  }
  const size_t nwords = (P.total - P.xbuf) / 8;
  decode_persistent_init_kernel<<<256, 256, 0, st>>>(a.hdr, a.xbuf, nwords);
  decode_persistent_mark_kernel<<<1, 64, 0, st>>>(a.hdr);
  const int mt = T == 1 ? 1 : T == 2 ? 2 : 4;
  const int slots = E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16;
  const void* fn = nullptr;
#define PT_PICK(Q, M, S) \
  if (qfmt == Q && mt == M && slots == S) fn = (const void*)decode_persistent_kernel<Q, M, S>;
#define PT_PICK_S(Q, M) PT_PICK(Q, M, 1) PT_PICK(Q, M, 2) PT_PICK(Q, M, 4) PT_PICK(Q, M, 8) PT_PICK(Q, M, 16)
  PT_PICK_S(MOE_Q4_B32, 1) PT_PICK_S(MOE_Q4_B32, 2) PT_PICK_S(MOE_Q4_B32, 4)
  PT_PICK_S(MOE_Q2_B16, 1) PT_PICK_S(MOE_Q2_B16, 2) PT_PICK_S(MOE_Q2_B16, 4)
#undef PT_PICK_S
#undef PT_PICK
  if (!fn) return moe_fail(MOE_EUNSUPPORTED, "decode persistent: no kernel for this shape");
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)P.lds) != hipSuccess)
    return moe_fail(MOE_EHIP, "decode persistent: cannot reserve %zu bytes of LDS", P.lds);
  void* args[] = {&a};
  if (hipLaunchKernel(fn, dim3(G), dim3(PT_THREADS), args, P.lds, st) != hipSuccess)
    return moe_fail(MOE_EHIP, "decode persistent: launch failed");
  return moe_check_launch("decode persistent");
}
