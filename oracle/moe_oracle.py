"""CPU oracle of the routed-expert MoE-FFN layer -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this module.  It shares no code with the HIP library (routed_expert_ffn_moe_amd)
and imports nothing from it.  Everything is computed in fp64 NumPy, written
for a reader to check against the definitions by eye; it is deliberately slow.

What it follows (pages about the Strata engine for Qwen3.8-Flash-Next):
  * "Strata开源运行时：12GB显卡跑动125B参数Qwen3模型", section
    "模型本身：稀疏MoE带来的计算与存储鸿沟": per layer a router selects 10 of
    512 experts per token and one shared expert always runs; the FFN is split
    into parallel expert sub-networks chosen by a light router.
  * "为什么 Strata 在小显存显卡上这么快", section "问题：1250 亿参数，12 GB
    显存": 48 layers x 512 experts, 10 per layer per token.
  * same page, section "一个 token，三路工人": the GPU sums the experts'
    results, then the next layer starts.
  * same page, section "由粗到细": the adaptive tier swaps in at most 96
    experts every four rounds; "Strata：12GB 显卡跑 125B 模型，MoE 专家热缓存
    打破 VRAM 限制", section "工作原理": eviction follows an exponentially
    decayed usage score.
Where the pages are silent, the readings are the ones stated in include/moe.h
(SwiGLU experts, softmax over the chosen logits, ties to the lower index,
shared expert with weight 1, the record byte format, and a stack of layers
as a pre-norm residual chain x_{l+1} = x_l + MoE_l(x_l / rms(x_l))).

Pins: every function here is checked in tests/test_oracle_pins.py against
hand-derived values, closed forms, brute force or library routines.  No
function is left "parity unpinned".
"""
import numpy as np

__all__ = [
    "bf16_to_f64", "f16_to_f64", "decode_record", "expert_getter",
    "router_logits", "topk_select", "topk_gaps", "gap_ok", "silu",
    "expert_ffn", "moe_layer", "combine", "permute", "usage_update",
    "moe_stack_decode", "rms_normalize",
]

QFMT_INT4 = 0
QFMT_INT2 = 1


# ----------------------------------------------------------------------------
# number formats

def bf16_to_f64(bits):
    """bf16 bit patterns (any int dtype) -> float64 (exact widening)."""
    b = np.asarray(bits).astype(np.uint32) & 0xFFFF
    return (b << 16).view(np.float32).astype(np.float64)


def f16_to_f64(bits):
    b = np.asarray(bits).astype(np.uint16)
    return b.view(np.float16).astype(np.float64)


# ----------------------------------------------------------------------------
# record decoding (byte format of include/moe.h, "Expert weight records")

def _words(rec, start, nbytes):
    return np.frombuffer(np.ascontiguousarray(rec[start:start + nbytes]).tobytes(), dtype="<u4")


def _halves(rec, start, nbytes):
    return np.frombuffer(np.ascontiguousarray(rec[start:start + nbytes]).tobytes(), dtype="<u2")


def _int4_matrix(rec, q_off, s_off, rows, K, grouped_scales):
    """Decode one int4 plane pair into a dense fp64 [rows][K] matrix.  Scales
    are stored [kb/4][row][4] (grouped) or [kb][row]."""
    KB = K // 32
    w = _words(rec, q_off, rows * K // 2).reshape(KB, rows, 4)   # [kb][row][word j]
    vals = np.empty((KB, rows, 4, 8), dtype=np.int64)            # value 8j+v
    for i in range(4):
        vals[..., 2 * i] = (w >> (4 * i)) & 0xF
        vals[..., 2 * i + 1] = (w >> (16 + 4 * i)) & 0xF
    q = vals.reshape(KB, rows, 32).transpose(1, 0, 2) - 8          # [row][kb][32]
    if grouped_scales:
        s = f16_to_f64(_halves(rec, s_off, rows * KB * 2).reshape(KB // 4, rows, 4))
        s = s.transpose(1, 0, 2).reshape(rows, KB)                 # [row][kb]
    else:
        s = f16_to_f64(_halves(rec, s_off, rows * KB * 2).reshape(KB, rows)).T
    return (q * s[:, :, None]).reshape(rows, K)


def _int2_block_values(w):
    """words [...] of one int2 block each -> values [..., 16]."""
    vals = np.empty(w.shape + (16,), dtype=np.int64)
    for i in range(8):
        vals[..., 2 * i] = (w >> (2 * i)) & 0x3
        vals[..., 2 * i + 1] = (w >> (16 + 2 * i)) & 0x3
    return vals


def _int2_matrix(rec, q_off, m_off, rows, K, grouped):
    """Decode one int2 plane pair into a dense fp64 [rows][K] matrix.  Words
    and (s, m) pairs are stored in 4-block units [K/64][row][4] (grouped) or
    per block [K/16][row]."""
    NB = K // 16
    if grouped:
        w = _words(rec, q_off, rows * K // 4).reshape(NB // 4, rows, 4)   # word j = block 4u+j
        q = _int2_block_values(w).transpose(1, 0, 2, 3).reshape(rows, NB, 16)
        meta = f16_to_f64(_halves(rec, m_off, rows * NB * 4).reshape(NB // 4, rows, 4, 2))
        meta = meta.transpose(1, 0, 2, 3).reshape(rows, NB, 2)
    else:
        w = _words(rec, q_off, rows * K // 4).reshape(NB, rows)
        q = _int2_block_values(w).transpose(1, 0, 2)                      # [row][block][16]
        meta = f16_to_f64(_halves(rec, m_off, rows * NB * 4).reshape(NB, rows, 2)).transpose(1, 0, 2)
    s, m = meta[..., 0], meta[..., 1]
    return (q * s[:, :, None] + m[:, :, None]).reshape(rows, K)


def decode_record(rec, qfmt, H, F):
    """One record -> (Wg [F][H], Wu [F][H], Wd [H][F]) in fp64."""
    rec = np.asarray(rec, dtype=np.uint8)
    HF = H * F
    if qfmt == QFMT_INT4:
        gu = _int4_matrix(rec, 0, 3 * HF // 2, 2 * F, H, grouped_scales=True)
        wd = _int4_matrix(rec, HF, 3 * HF // 2 + HF // 8, H, F, grouped_scales=False)
    elif qfmt == QFMT_INT2:
        gu = _int2_matrix(rec, 0, 3 * HF // 4, 2 * F, H, grouped=True)
        wd = _int2_matrix(rec, HF // 2, 5 * HF // 4, H, F, grouped=False)
    else:
        raise ValueError(qfmt)
    # GU row 64g+i is gate row 32g+i (i < 32) or up row 32g+i-32 (i >= 32)
    gu = gu.reshape(F // 32, 2, 32, H)
    wg = gu[:, 0].reshape(F, H)
    wu = gu[:, 1].reshape(F, H)
    return wg, wu, wd


def expert_getter(pool, slot_table, layer, qfmt, H, F, rec_bytes):
    """Callable e -> decoded (Wg, Wu, Wd) of expert e of `layer` (e == E is
    the shared expert).  `pool` is anything sliceable to uint8 bytes."""
    cache = {}
    S = np.asarray(slot_table)

    def get(e):
        if e not in cache:
            s = int(S[layer, e])
            cache[e] = decode_record(np.asarray(pool[s * rec_bytes:s * rec_bytes + rec_bytes]),
                                     qfmt, H, F)
        return cache[e]
    return get


# ----------------------------------------------------------------------------
# router and top-k

def router_logits(x, Wr, bias=None):
    """l[t,e] = sum_h x[t,h] Wr[e,h] (+ b[e]), fp64."""
    l = np.asarray(x, np.float64) @ np.asarray(Wr, np.float64).T
    if bias is not None:
        l = l + np.asarray(bias, np.float64)[None, :]
    return l


def topk_select(logits, k):
    """Top-k by (logit descending, expert index ascending) and the softmax of
    the chosen logits.  Returns (idx int64 [T][k], w fp64 [T][k])."""
    logits = np.asarray(logits, np.float64)
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int64)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t]))
        idx[t] = order[:k]
        z = np.exp(logits[t, idx[t]] - logits[t, idx[t, 0]])
        w[t] = z / z.sum()
    return idx, w


def topk_gaps(logits, k):
    """Smallest gap between adjacent values among each token's k+1 largest
    logits (k largest when k == E)."""
    srt = -np.sort(-np.asarray(logits, np.float64), axis=1)[:, :k + 1]
    if srt.shape[1] < 2:
        return np.full(srt.shape[0], np.inf)
    return (srt[:, :-1] - srt[:, 1:]).min(axis=1)


def gap_ok(logits, k, min_gap=1e-3):
    """Tokens whose top-k set and order are decided by a margin >= min_gap."""
    return topk_gaps(logits, k) >= min_gap


# ----------------------------------------------------------------------------
# experts

def silu(z):
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(Wg, Wu, Wd, x):
    """SwiGLU expert on rows of x: Wd (silu(Wg x) * (Wu x))."""
    x = np.asarray(x, np.float64)
    g = x @ Wg.T
    u = x @ Wu.T
    return (silu(g) * u) @ Wd.T


def combine(y_routed, w, y_shared, residual=None):
    """y[t] = sum_j w[t,j] y_routed[t,j] + y_shared[t] (+ residual[t])."""
    y = np.einsum("tj,tjh->th", w, y_routed) + y_shared
    if residual is not None:
        y = y + residual
    return y


def moe_layer(x, Wr, bias, k, get_expert, E):
    """One MoE layer on tokens x [T][H] (fp64).  get_expert(e) returns the
    dense (Wg, Wu, Wd) of routed expert e < E or of the shared expert e == E.
    Returns (y [T][H], idx [T][k], w [T][k], y_parts [T][k+1][H], logits)."""
    x = np.asarray(x, np.float64)
    T, H = x.shape
    logits = router_logits(x, Wr, bias)
    idx, w = topk_select(logits, k)
    y_parts = np.zeros((T, k + 1, H))
    for t in range(T):
        for j in range(k):
            y_parts[t, j] = expert_ffn(*get_expert(int(idx[t, j])), x[t:t + 1])[0]
        y_parts[t, k] = expert_ffn(*get_expert(E), x[t:t + 1])[0]
    y = combine(y_parts[:, :k], w, y_parts[:, k])
    return y, idx, w, y_parts, logits


def rms_normalize(x, eps=1e-6):
    """x / sqrt(mean(x^2) + eps) per token (unit gain)."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def moe_stack_decode(x, Wr_layers, bias_layers, k, getters, E, eps=1e-6):
    """Chain layers with a pre-norm residual: x_{l+1} = x_l + MoE_l(rms(x_l)).
    getters[l] is layer l's expert getter.  Returns (x_out, idx [L][T][k],
    w [L][T][k], x_hist [L][T][H]) where x_hist[l] is x_l (before the norm)."""
    x = np.asarray(x, np.float64)
    idxs, ws, hist = [], [], []
    for l, get in enumerate(getters):
        hist.append(x.copy())
        b = None if bias_layers is None else bias_layers[l]
        y, idx, w, _, _ = moe_layer(rms_normalize(x, eps), Wr_layers[l], b, k, get, E)
        idxs.append(idx)
        ws.append(w)
        x = x + y
    return x, np.array(idxs), np.array(ws), np.array(hist)


# ----------------------------------------------------------------------------
# permutation by expert (prefill)

def permute(idx, E):
    """Group the flat pairs t*k+j by expert, keeping ascending flat order
    inside each expert.  Returns (counts [E], offsets [E+1], row_src, inv_row)."""
    flat = np.asarray(idx).reshape(-1)
    row_src = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    inv_row = np.empty_like(row_src)
    inv_row[row_src] = np.arange(flat.size)
    return counts, offsets, row_src, inv_row


# ----------------------------------------------------------------------------
# usage counters

def usage_update(scores, idx, layer, decay, step, rerank_every, top_n):
    """Decayed usage of one layer, emulating fp32 exactly (one rounding per
    operation, no fused multiply-add).  Returns (new scores fp32 [L][E],
    top_out or None)."""
    s = np.array(scores, dtype=np.float32, copy=True)
    L, E = s.shape
    hits = np.zeros(E, dtype=np.int64)
    for row in np.asarray(idx):
        for e in set(int(v) for v in row):
            hits[e] += 1
    d = np.float32(decay)
    s[layer] = (s[layer] * d).astype(np.float32) + hits.astype(np.float32)
    top = None
    if layer == L - 1 and (step + 1) % rerank_every == 0:
        flat = s.reshape(-1).astype(np.float64)
        order = np.lexsort((np.arange(flat.size), -flat))
        top = order[:top_n]
    return s, top
