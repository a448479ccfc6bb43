/*
 * moe.h -- C ABI of the MI355X (gfx950) routed-expert MoE-FFN layer library
 * (libmoe.so).
 *
 * What the layer computes.  Pages describing the Strata engine for the
 * Qwen3.8-Flash-Next model:
 *   - "Strata开源运行时：12GB显卡跑动125B参数Qwen3模型", section
 *     "模型本身：稀疏MoE带来的计算与存储鸿沟": in every layer a router picks
 *     10 of 512 experts for each token, and one shared expert always runs;
 *     the model has 48 layers.
 *   - "为什么 Strata 在小显存显卡上这么快", section "问题：1250 亿参数，12 GB
 *     显存": 48 x 512 = 24,576 experts, 10 chosen per layer per token, so a
 *     token touches 480 routed experts.
 *   - same page, section "一个 token，三路工人": after the router, the chosen
 *     experts' results are summed on the GPU before the next layer starts.
 *   - same page, section "读长提示词：大块流式读取": prompts are read in
 *     chunks of up to 8,192 (or 16,384) tokens, and a chunk routes to nearly
 *     every expert of a layer.
 * The pages do not spell out the expert network or the quantisation; this
 * library fixes them as follows (all are part of the contract below):
 *   router   l[t,e] = sum_h x[t,h] * Wr[e,h] + b[e]       (fp32 accumulation)
 *   top-k    the k largest l[t,.], larger logit first, equal logits broken
 *            towards the lower expert index; w[t,j] = softmax over the k
 *            chosen logits (sums to 1).
 *   expert   SwiGLU: y_e(x) = Wd_e ( silu(Wg_e x) * (Wu_e x) ),
 *            silu(z) = z / (1 + exp(-z)).
 *   layer    y[t] = sum_{j<k} w[t,j] * y_{idx[t,j]}(x_t) + y_shared(x_t)
 *            (shared expert weight 1), summed in the order j = 0..k-1, then
 *            the shared expert.  A stack of layers is a pre-norm residual
 *            chain (see moe_decode_stack).
 *
 * ---------------------------------------------------------------------------
 * Conventions (all entry points)
 *   - Every data pointer is DEVICE memory owned by the caller.  The library
 *     never allocates, frees or retains device memory.  Scratch memory is the
 *     caller's `ws` buffer of `ws_bytes` bytes, sized by moe_workspace_size().
 *   - Work is enqueued asynchronously on the caller's HIP stream `stream`
 *     (a hipStream_t passed as void*; NULL = the null stream).  No entry point
 *     synchronises the device.
 *   - Return value: MOE_OK (0) or a negative MOE_E* code.  On error nothing
 *     has been enqueued and moe_last_error() (thread-local) describes it.
 *     Arguments are validated on the host before any launch.  Index contents
 *     of device arrays (expert ids, slots, rows) are preconditions that are
 *     not read on the host; an out-of-range value is undefined behaviour.
 *     The moe_validate_* functions (end of this file) check such arrays
 *     once the caller has copied them to host memory.
 *   - bf16 and fp16 values are passed as uint16_t bit patterns.
 *   - Entry points keep no state between calls: calls on different streams
 *     with different workspaces may run concurrently.
 *   - Results are deterministic: no floating-point atomics are used, so a
 *     repeated call on the same inputs gives bit-identical outputs.
 *
 * ---------------------------------------------------------------------------
 * Expert weight records
 *   One expert = gate Wg [F][H], up Wu [F][H], down Wd [H][F] (row-major
 *   [out][in]).  Quantisation blocks run along the input (K) dimension.
 *   Shapes must satisfy H % 128 == 0 and F % 128 == 0.
 *
 *   The gate and up matrices are stored as one "GU" matrix of 2F rows:
 *   GU row r, with g = r / 64 and i = r % 64, is gate row 32g+i when i < 32
 *   and up row 32g+i-32 otherwise (gate and up alternate in runs of 32 rows).
 *   The down matrix is stored as its H rows.
 *
 *   MOE_Q4_B32 (qfmt 0): blocks of 32 values, each with one fp16 scale s;
 *   value = s * q, q in [-8, 7], stored as the nibble q + 8.
 *     A 16-byte block holds four little-endian 32-bit words; word j holds
 *     block values 8j..8j+7: value 8j+2i in bits [4i, 4i+4) and value 8j+2i+1
 *     in bits [16+4i, 16+4i+4), i = 0..3.
 *     Planes of one record (byte offsets from the record start):
 *       GU_Q  at 0           : block (kb, r), kb < H/32, r < 2F, at 16*(kb*2F + r)
 *       D_Q   at H*F         : block (kb, r), kb < F/32, r < H,  at 16*(kb*H + r)
 *       GU_S  at 3HF/2       : scale (kb, r) at 2*((kb/4)*2F*4 + 4r + kb%4)
 *       D_S   at 3HF/2+HF/8  : scale (kb, r) at 2*(kb*H + r)
 *     Record size 27HF/16 bytes (2,654,208 B at H=2048, F=768).
 *
 *   MOE_Q2_B16 (qfmt 1): blocks of 16 values, each with an fp16 scale s and an
 *   fp16 offset m; value = s * q + m, q in [0, 3] stored as 2 bits.
 *     A 32-bit little-endian word holds one block: value 2i in bits
 *     [2i, 2i+2) and value 2i+1 in bits [16+2i, 16+2i+2), i = 0..7.
 *     A 16-byte q-unit holds 4 consecutive blocks (word j = block 4u+j).
 *     A 16-byte meta-unit holds (s, m) of 4 consecutive blocks: block 4u+j's
 *     s at byte 4j and m at byte 4j+2.  The down planes are not grouped.
 *       GU_Q  at 0           : q-unit (u, r), u < H/64, at 16*(u*2F + r)
 *       D_Q   at HF/2        : word of block (b, r), b < F/16, r < H, at 4*(b*H + r)
 *       GU_M  at 3HF/4       : meta-unit (u, r), u < H/64, at 16*(u*2F + r)
 *       D_M   at 5HF/4       : (s, m) of block (b, r) at 4*(b*H + r), m at +2
 *     Record size 3HF/2 bytes (2,359,296 B at H=2048, F=768).
 *
 *   Pool and slot table.  All records live in one caller-owned pool; the
 *   record in slot s starts at pool + s * record_bytes.  pool must be 256-byte
 *   aligned; record_bytes must be a multiple of 256 and at least
 *   moe_record_bytes(qfmt, H, F).  The slot table S is int32 [L][E+1]:
 *   S[l][e] is the slot of routed expert e of layer l, S[l][E] the slot of
 *   layer l's shared expert.
 *
 *   Router weights Wr are bf16 [E][H] row-major per layer ([L][E][H] for a
 *   stack); the optional bias b is fp32 [E] per layer ([L][E] for a stack).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

/* return codes */
#define MOE_OK            0
#define MOE_EINVAL       (-1) /* null pointer or meaningless argument      */
#define MOE_ESHAPE       (-2) /* size outside the supported range          */
#define MOE_EALIGN       (-3) /* misaligned pointer or record size         */
#define MOE_EUNSUPPORTED (-4) /* unknown dtype / format / op               */
#define MOE_EWORKSPACE   (-5) /* ws too small (or NULL when needed)        */
#define MOE_EHIP         (-6) /* the HIP runtime reported a launch error    */

/* activation dtypes */
#define MOE_F32  0
#define MOE_BF16 1
#define MOE_F16  2  /* expert output rows of the prefill path */

/* weight formats */
#define MOE_Q4_B32 0
#define MOE_Q2_B16 1

/* op ids for moe_workspace_size */
#define MOE_OP_ROUTE_TOPK     0
#define MOE_OP_PERMUTE        1
#define MOE_OP_EXPERT_GEMV_Q  2
#define MOE_OP_GROUPED_GEMM_Q 3
#define MOE_OP_COMBINE        4
#define MOE_OP_USAGE_UPDATE   5
#define MOE_OP_DECODE_STACK   6

/* Supported ranges (checked on the host). */
#define MOE_MAX_E        1024  /* routed experts per layer                  */
#define MOE_MAX_K        16    /* top-k                                     */
#define MOE_MAX_DECODE_T 8     /* tokens per decode / verify call           */
#define MOE_MAX_H        8192
#define MOE_MAX_F        8192

/* Version of this ABI (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Thread-local description of the last error returned on this thread
 * ("" if none).  The string stays valid until the next call on the thread. */
const char* moe_last_error(void);

/* Minimum record size in bytes for format qfmt (0 if the shape or format is
 * unsupported). */
int64_t moe_record_bytes(int qfmt, int H, int F);

/* Workspace bytes that entry point `op` needs for these sizes (0 = none).
 * Arguments that an op does not use are ignored (pass 0).  For
 * MOE_OP_DECODE_STACK, F is the FFN size and E the routed expert count;
 * the layer count does not change the size.  Returns 0 for unknown ops. */
size_t moe_workspace_size(int op, int T, int k, int E, int H, int F, int qfmt);

/* --------------------------------------------------------------------------
 * moe_route_topk -- router logits, top-k selection and softmax weights.
 * Pages: "Strata开源运行时：12GB显卡跑动125B参数Qwen3模型", section
 * "模型本身：稀疏MoE带来的计算与存储鸿沟" (in every layer a light router
 * picks 10 of the 512 experts for each token); "为什么 Strata 在小显存显卡上
 * 这么快", section "一个 token，三路工人" (per layer the GPU runs the router
 * first and the ids of the 10 chosen experts decide where the work goes).
 *   x        [T][H] activations, dtype x_dtype (MOE_F32 or MOE_BF16)
 *   w_router bf16 [E][H], bias fp32 [E] or NULL
 *   topk_idx int32 [T][k] out: chosen experts, larger logit first, ties to
 *            the lower index
 *   topk_w   fp32 [T][k] out: softmax of the chosen logits
 *   logits_out fp32 [T][E] out, or NULL (the logits then go to ws)
 * Requires 1 <= k <= MOE_MAX_K, k <= E <= MOE_MAX_E, H % 128 == 0, T >= 0.
 * A NaN logit is a caller error (the choice is then unspecified).
 * ws: moe_workspace_size(MOE_OP_ROUTE_TOPK, T, k, E, H, 0, 0) bytes; may be
 * NULL when logits_out is given. */
int moe_route_topk(const void* x, int x_dtype, int T, int H,
                   const uint16_t* w_router, const float* bias, int E, int k,
                   int32_t* topk_idx, float* topk_w, float* logits_out,
                   void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------
 * moe_permute -- group the T*k (token, choice) pairs by expert; stable.
 * Page: "为什么 Strata 在小显存显卡上这么快", section "读长提示词：大块流式
 * 读取" (a prompt is read in chunks of up to 8,192 or 16,384 tokens; such a
 * chunk routes to nearly every expert of a layer and each expert's weights
 * then serve all of the chunk's tokens that chose it -- grouping the pairs
 * by expert is what lets one pass over an expert serve all of them).
 *   counts  int32 [E]   out: counts[e] = #{(t,j) : topk_idx[t][j] == e}
 *   offsets int32 [E+1] out: exclusive prefix sum, offsets[E] = T*k
 *   row_src int32 [T*k] out: row_src[r] = t*k+j of the pair placed at row r;
 *           rows of one expert keep ascending t*k+j order
 *   inv_row int32 [T*k] out: inv_row[row_src[r]] = r
 *   x_perm  optional [T*k][H] out (dtype x_dtype): x_perm[r] = x[row_src[r]/k]
 *           (pass x = x_perm = NULL to skip)
 * Requires 1 <= k <= MOE_MAX_K, k <= E <= MOE_MAX_E, T*k < 2^31, and
 * topk_idx entries in [0, E).  ws: moe_workspace_size(MOE_OP_PERMUTE, ...). */
int moe_permute(const int32_t* topk_idx, int T, int k, int E,
                int32_t* counts, int32_t* offsets, int32_t* row_src,
                int32_t* inv_row, const void* x, int x_dtype, int H,
                void* x_perm, void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------
 * moe_expert_gemv_q -- decode / verify experts (1 <= T <= MOE_MAX_DECODE_T).
 * Pages: "为什么 Strata 在小显存显卡上这么快", section "一个 token，三路工人"
 * (the chosen experts of each layer are computed, then summed on the GPU);
 * same page, section "先猜，再检查" (a verify step of several tokens reads
 * the shared weights once, and only experts that the extra tokens route to
 * add work -- hence each distinct expert is read once per call);
 * "Strata开源运行时：12GB显卡跑动125B参数Qwen3模型", section "模型本身：稀疏
 * MoE带来的计算与存储鸿沟" (10 routed experts plus one shared expert that
 * always runs).
 *   x        fp32 [T][H]
 *   topk_idx int32 [T][k] (from moe_route_topk)
 *   y_parts  fp32 [T][k+1][H] out: y_parts[t][j] = y_{topk_idx[t][j]}(x_t)
 *            for j < k, y_parts[t][k] = y_shared(x_t); not weighted.
 * Each distinct expert of the call is read from the pool once.
 * ws: moe_workspace_size(MOE_OP_EXPERT_GEMV_Q, T, k, E, H, F, qfmt). */
int moe_expert_gemv_q(const float* x, int T, int H, int F,
                      const int32_t* topk_idx, int k, int E,
                      const int32_t* slot_table, int layer, const void* pool,
                      int64_t record_bytes, int qfmt, float* y_parts,
                      void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------
 * moe_grouped_gemm_q -- prefill experts over a permuted chunk.
 * Page: "为什么 Strata 在小显存显卡上这么快", section "读长提示词：大块流式
 * 读取" (every expert a chunk routes to is used by the whole chunk, so its
 * weight traffic is amortised over thousands of tokens: a dense contraction
 * per expert); "Strata开源运行时：12GB显卡跑动125B参数Qwen3模型", section
 * "模型本身：稀疏MoE带来的计算与存储鸿沟" (the shared expert always runs).
 *   x        bf16 [T][H]; every |x| must be below 65520 (fp16's range)
 *   row_src, offsets: from moe_permute (rows of expert e are
 *            [offsets[e], offsets[e+1]))
 *   y_perm   [T*k][H] out, dtype y_dtype: y_perm[r] = y_e(x[row_src[r]/k])
 *   y_shared [T][H]   out, dtype y_dtype: y_shared[t] = y_shared(x[t])
 *            (x, y_perm and y_shared 16-byte aligned, else MOE_EALIGN)
 *   y_dtype  MOE_F32, or MOE_F16 (one rounding of the fp32 sum; half the
 *            bytes written here and read by moe_combine; |y| >= 65520
 *            becomes inf, not checked)
 * Experts with no rows are skipped.  Internally x is multiplied in fp16:
 * bf16 values with 2^-14 <= |x| < 65520 convert exactly; smaller ones round
 * to fp16 subnormals (absolute error <= 2^-25); |x| >= 65520 becomes inf
 * (not checked: the output is then inf/NaN for the tokens concerned).
 * Weights are dequantised to fp16 (one rounding of s*q, resp. s*q+m), the
 * SiLU*mul intermediate is rounded to fp16 and all sums are fp32.
 * ws: moe_workspace_size(MOE_OP_GROUPED_GEMM_Q, T, k, E, H, F, qfmt). */
int moe_grouped_gemm_q(const uint16_t* x, int T, int H, int F,
                       const int32_t* row_src, const int32_t* offsets, int k,
                       int E, const int32_t* slot_table, int layer,
                       const void* pool, int64_t record_bytes, int qfmt,
                       void* y_perm, void* y_shared, int y_dtype, void* ws,
                       size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------
 * moe_combine -- weighted sum of the expert outputs of each token.
 * Page: "为什么 Strata 在小显存显卡上这么快", section "一个 token，三路工人"
 * (the GPU adds up the experts' results before the next layer starts).
 *   inv_row == NULL: decode layout, y_rows is [T][k+1][H] as written by
 *     moe_expert_gemv_q (slot k = shared expert) and y_shared must be NULL.
 *   inv_row != NULL: prefill layout, y_rows is y_perm [T*k][H] and y_shared
 *     is [T][H].
 *   rows_dtype: MOE_F32 or MOE_F16, the dtype of y_rows and y_shared (fp16
 *     as moe_grouped_gemm_q writes them with y_dtype = MOE_F16).
 *   y_out[t] = sum_{j<k} topk_w[t][j] * row(t,j) + shared(t) (+ residual[t])
 *   summed in that order in fp32.  residual may be NULL; y_out may alias
 *   residual.
 */
int moe_combine(const void* y_rows, int rows_dtype, const int32_t* inv_row,
                const void* y_shared, const float* topk_w,
                const float* residual, int T, int k, int H, float* y_out,
                void* stream);

/* --------------------------------------------------------------------------
 * moe_usage_update -- per-step expert usage with exponential decay and a
 * periodic global re-rank.  Pages: "Strata：12GB 显卡跑 125B 模型，MoE 专家
 * 热缓存打破 VRAM 限制", section "工作原理" (exponential decay: the more an
 * expert is used the harder it is to evict); "为什么 Strata 在小显存显卡上
 * 这么快", section "由粗到细" (the adaptive tier swaps in at most 96 experts
 * every four rounds).
 *   hits[e]  = number of the T tokens whose topk_idx row contains e
 *   scores[layer][e] <- fp32( fp32(decay * scores[layer][e]) + hits[e] ),
 *              for every e < E, each operation rounded to fp32 (no FMA)
 *   When layer == L-1, top_out != NULL and (step+1) % rerank_every == 0:
 *   top_out[i] = flat index l*E+e of the i-th largest score over all L*E
 *   entries, larger score first, equal scores by lower flat index.
 *   hits_ws  int32 [E] scratch (device).
 * Requires scores >= 0 and finite, 1 <= top_n <= min(L*E, 1024),
 * L*E <= 65536, rerank_every >= 1. */
int moe_usage_update(const int32_t* topk_idx, int T, int k, int layer, int L,
                     int E, float decay, int64_t step, int rerank_every,
                     int top_n, int32_t* hits_ws, float* scores,
                     int32_t* top_out, void* stream);

/* moe_usage_update_stack -- the same for every layer of a step at once:
 * exactly moe_usage_update(topk_idx + l*T*k, T, k, l, L, E, decay, step,
 * rerank_every, top_n, hits_ws + l*E, scores, top_out) for l = 0..L-1 in
 * order, in one launch (one workgroup per layer) plus the re-rank.
 *   topk_idx int32 [L][T][k] (as moe_decode_stack's topk_idx_out);
 *   hits_ws  int32 [L][E] scratch (device). */
int moe_usage_update_stack(const int32_t* topk_idx, int T, int k, int L, int E,
                           float decay, int64_t step, int rerank_every,
                           int top_n, int32_t* hits_ws, float* scores,
                           int32_t* top_out, void* stream);

/* --------------------------------------------------------------------------
 * Capacity-limited hot tier of expert records.  Pages: "为什么 Strata 在小显存
 * 显卡上这么快", section "一台电脑就是一组水管" (a shipped usage profile ranks
 * every expert and each card fills its expert slots in that order; an
 * adaptive tier swaps in at most 96 experts every four rounds, towards the
 * experts in actual use); "Strata：12GB 显卡跑 125B 模型，MoE 专家热缓存打破
 * VRAM 限制", section "工作原理" (a decayed usage score decides eviction).
 *
 * Layout: pool holds n_hot hot slots (slots 0..n_hot-1) followed by every
 * expert's record at its home slot, home_table int32 [L][E+1] (every home slot
 * >= n_hot, distinct; column E, the shared expert, is never part of the
 * tier).  slot_table int32 [L][E+1] is what the expert ops and
 * moe_decode_stack read: a resident expert's entry is its hot slot, every
 * other entry equals home_table.  hot_owner int32 [n_hot] holds the flat index
 * l*E+e of the expert in each hot slot, or -1 (empty).  Records are copied on
 * the device with 16-byte loads and stores; record_bytes is a multiple of 256
 * and pool 256-byte aligned.  swaps int32 [max(n_hot, max_swaps)][4] receives
 * one entry per copied record: (expert, evicted expert or -1, hot slot, home
 * slot of the expert); n_swaps int32 [1] their count.  All device memory,
 * owned by the caller; asynchronous on `stream`.  Requires L*E <= 65536,
 * 1 <= n_hot <= L*E, finite scores.  A call that overlaps another tier call
 * or a reader of the same slot table on another stream races.
 *
 * moe_tier_fill -- resets the tier from a profile: slot_table = home_table,
 *   then the n_hot experts first in the order (scores desc, flat index asc)
 *   become resident, hot slot i holding the i-th of them in flat-index order.
 *   scores fp32 [L][E] (e.g. the scores of moe_usage_update).
 *
 * moe_tier_rebalance -- one adaptive step (e.g. every fourth decode step,
 *   max_swaps = 96).  Candidates: the experts that are not resident, in the
 *   order (scores desc, flat index asc).  Victims: the hot slots, empty ones
 *   first (lower slot first), then by the held expert's score ascending,
 *   equal scores the higher flat index first.  Candidate i takes victim i's
 *   slot while that slot is empty or the candidate's score is strictly higher
 *   (equal scores never swap), at most max_swaps times; an evicted expert's
 *   entry returns to its home slot.  0 <= max_swaps <= 1024. */
int moe_tier_fill(const float* scores, int L, int E, int n_hot,
                  const int32_t* home_table, int32_t* slot_table,
                  int32_t* hot_owner, void* pool, int64_t record_bytes,
                  int32_t* swaps, int32_t* n_swaps, void* stream);
int moe_tier_rebalance(const float* scores, int L, int E, int n_hot,
                       int max_swaps,
                       const int32_t* home_table, int32_t* slot_table,
                       int32_t* hot_owner, void* pool, int64_t record_bytes,
                       int32_t* swaps, int32_t* n_swaps, void* stream);

/* --------------------------------------------------------------------------
 * moe_decode_stack -- one decode / verify step through L chained layers
 * (1 <= T <= MOE_MAX_DECODE_T), the whole step enqueued on `stream` with no
 * host synchronisation (it may be captured into a HIP graph).  Pages: "为什么 Strata 在小显存显卡上这么快", section
 * "一个 token，三路工人" (the whole 48-layer forward is recorded once and
 * replayed so that the host never waits inside a step); section "先猜，再检查"
 * (a verify step runs 1 real + up to 3 drafted tokens through all 48 layers).
 *   x_in     fp32 [T][H];  x_out fp32 [T][H] (may not alias x_in)
 *   w_router bf16 [L][E][H];  bias fp32 [L][E] or NULL
 *   slot_table int32 [L][E+1]
 *   topk_idx_out int32 [L][T][k] or NULL; topk_w_out fp32 [L][T][k] or NULL
 *   x_hist   fp32 [L][T][H] or NULL: x_hist[l] = x_l, the residual stream
 *            entering layer l
 * Layers chain as a pre-norm residual stream (the pages do not describe the
 * non-MoE parts of a layer; without a norm a chain of SwiGLU layers, which
 * are quadratic in x, overflows within a few layers):
 *   xn_l = x_l / sqrt(mean_h(x_l^2) + 1e-6)          (unit gain)
 *   x_{l+1} = x_l + MoE_l(xn_l)
 * where MoE_l(xn_l) is exactly what moe_route_topk + moe_expert_gemv_q +
 * moe_combine compute on xn_l with layer l's router, bias and slots.
 * Execution: for 1 <= T <= 8 (and shapes whose working set
 * fits in LDS) the step runs as ONE persistent kernel whose workgroups pass
 * data through tagged words in ws (no host synchronisation, no grid
 * barrier); otherwise,
 * or when the environment variable MOE_DECODE_PATH=chain is set, as a chain
 * of kernels per layer.  The persistent path is taken only when the device
 * reports that all its workgroups (one per CU) fit at once.
 * Workspace: the persistent path keeps a header (a count of the exchange
 * tags used so far, with check words) and tagged exchange buffers in ws
 * across calls.  Every call uses tags no earlier call on the same ws used,
 * so a ws may serve any sequence of calls (any L, T, k) as long as nothing
 * else writes it in between and calls on one ws do not overlap.  A ws whose
 * header is not valid (first use; memory that held other data) is zeroed
 * in full before use; passing zero-filled memory the first time is the
 * recommended practice.  The waits are bounded; if one times out (e.g.
 * other work on the device kept some workgroups from starting) x_out is
 * filled with NaN and the next call on that ws zeroes it first.
 * ws: moe_workspace_size(MOE_OP_DECODE_STACK, T, k, E, H, F, qfmt). */
int moe_decode_stack(const float* x_in, int T, int H, int F, int E, int k,
                     int L, const uint16_t* w_router, const float* bias,
                     const int32_t* slot_table, const void* pool,
                     int64_t record_bytes, int qfmt, float* x_out,
                     int32_t* topk_idx_out, float* topk_w_out, float* x_hist,
                     void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------
 * moe_rmsnorm -- the pre-norm of a stack of layers (see moe_decode_stack):
 *   out[t][h] = x[t][h] / sqrt(mean_h(x[t]^2) + eps)   (unit gain)
 * x fp32 [T][H]; out [T][H] in out_dtype: MOE_F32, or MOE_BF16 (each value
 * rounded once, to nearest even) to feed a prefill chunk's moe_route_topk and
 * moe_grouped_gemm_q.  Sums in fp32 in a fixed order.  out may not alias x.
 * With moe_combine(..., residual = x, y_out = x) this chains a prefill chunk
 * through the layers of a stack exactly as moe_decode_stack chains a decode
 * step. */
int moe_rmsnorm(const float* x, int T, int H, float eps, void* out, int out_dtype, void* stream);

/* --------------------------------------------------------------------------
 * moe_decode_stack_noalloc -- moe_decode_stack (same arguments, same
 * results, same kernels) without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Its scratch is a
 * library-owned device array of MOE_NOALLOC_WS_BYTES bytes, one per GPU the
 * library runs on, held until the process ends; the entry point allocates
 * nothing (no hipMalloc, no allocating library call).  Sizes whose
 * moe_workspace_size(MOE_OP_DECODE_STACK, ...) exceeds MOE_NOALLOC_WS_BYTES
 * are rejected with MOE_EWORKSPACE before anything is enqueued (at H = 2048,
 * E = 512, k = 10: T <= 5 fits, i.e. decode and verify windows of up to 4
 * drafted tokens; T = 6 and 8 need 26.9 and 35.9 MB and are rejected).
 * Every call on a GPU shares that GPU's array, which keeps the previous
 * call's contents (its tag header is valid
 * across calls; see moe_decode_stack): calls that overlap on one GPU, on
 * any streams, race and give wrong results.  The first call on a device
 * looks up the array's address (hipGetSymbolAddress) with that device
 * current. */
#define MOE_NOALLOC_WS_BYTES (24 << 20)
int moe_decode_stack_noalloc(const float* x_in, int T, int H, int F, int E, int k, int L,
                             const uint16_t* w_router, const float* bias, const int32_t* slot_table,
                             const void* pool, int64_t record_bytes, int qfmt, float* x_out,
                             int32_t* topk_idx_out, float* topk_w_out, float* x_hist, void* stream);

/* --------------------------------------------------------------------------
 * Host-side index checks.  The entry points above take the index contents
 * of their device arrays (expert ids, slots, rows) as preconditions and do
 * not read them on the host; these functions check such arrays after the
 * caller has copied them to HOST memory (a debugging aid: the Python
 * binding runs them before every call when MOE_VALIDATE=1).  They touch no
 * device.  Return MOE_OK, or MOE_EINVAL with moe_last_error() naming the
 * first offending entry (MOE_ESHAPE for impossible sizes).
 *
 * moe_validate_routing -- topk_idx int32 [T][k]: every id in [0, E) and the
 *   k ids of each token distinct (what moe_route_topk produces; required by
 *   moe_permute, moe_expert_gemv_q and moe_usage_update).
 * moe_validate_slot_table -- slot_table int32 [L][E+1]: every slot in
 *   [0, n_slots), n_slots being the number of records the pool holds.
 * moe_validate_rows -- offsets int32 [E+1], row_src int32 [n], inv_row
 *   int32 [n] or NULL, n = T*k: offsets[0] = 0, non-decreasing, offsets[E]
 *   = n; row_src a permutation of 0..n-1; inv_row its inverse (what
 *   moe_permute produces; required by moe_grouped_gemm_q and moe_combine). */
int moe_validate_routing(const int32_t* topk_idx, int T, int k, int E);
int moe_validate_slot_table(const int32_t* slot_table, int L, int E, int64_t n_slots);
int moe_validate_rows(const int32_t* offsets, const int32_t* row_src, const int32_t* inv_row, int T, int k,
                      int E);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
