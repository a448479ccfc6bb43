"""Seeded input generators and the record packer.

Recipe (every draw is seeded; the same call on the same device gives the same
tensor):
  x         fp32 ~ N(0, 1); prefill activations are that value rounded to bf16
  Wr        router weights ~ N(0, 0.05), rounded once to bf16, [E][H] per layer
  bias      optional popularity term b_e = ln p_e, p_e proportional to
            rank_e^-s (Zipf, s = 1.1), rank a seeded permutation of 1..E
  experts   Wg, Wu [F][H] and Wd [H][F] ~ N(0, 0.02), then quantised:
            int4: per block of 32 along the input dim, s = fp16(max|w| / 7),
                  q = clamp(round_half_even(w / s), -8, 7)
            int2: per block of 16, m = fp16(min w), s = fp16((max w - min w)/3),
                  q = clamp(round_half_even((w - m) / s), 0, 3)
            (a block whose scale is 0 gets q = 0, resp. q = 0)
  pool      one uint8 tensor of n_slots * record_bytes; the record of
            (layer l, expert e) sits at slot S[l][e], S a seeded permutation,
            column E of S being the shared expert.

Random numbers come from torch generators: on the CPU for small cases and on
the GPU for the large pools (the two devices give different streams for the
same seed; every test states where its inputs were drawn).
"""
import numpy as np
import torch

__all__ = [
    "QFMT_INT4", "QFMT_INT2", "record_bytes", "seed_of", "make_gen",
    "normal", "draw_x", "draw_x_rejecting", "to_bf16_bits", "draw_router",
    "zipf_bias", "quantize_int4", "quantize_int2", "pack_int4", "pack_int2",
    "pack_record", "draw_expert_weights", "make_slot_table", "build_pool",
    "LayerInputs", "make_layer_inputs", "draw_expert_chunks", "random_records", "build_random_pool",
]

QFMT_INT4 = 0
QFMT_INT2 = 1
EXPERT_CHUNK = 16  # experts drawn per generator call (part of the recipe)


def record_bytes(qfmt, H, F):
    """Bytes of one expert record (include/moe.h, "Expert weight records")."""
    if qfmt == QFMT_INT4:
        return 27 * H * F // 16
    if qfmt == QFMT_INT2:
        return 3 * H * F // 2
    raise ValueError(qfmt)


def seed_of(*parts):
    """A 63-bit seed from a tuple of ints / strings (numpy SeedSequence)."""
    ints = []
    for p in parts:
        if isinstance(p, str):
            ints.extend(p.encode())
        else:
            ints.append(int(p))
    st = np.random.SeedSequence(ints).generate_state(2, dtype=np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


def make_gen(device, *parts):
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*parts))
    return g


def normal(shape, std, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def to_bf16_bits(t):
    """fp32 -> bf16 (round to nearest even) bit patterns as int16."""
    return t.to(torch.bfloat16).view(torch.int16)


def draw_x(seed, T, H, device="cpu", tag="x", attempt=0):
    g = make_gen(device, seed, tag, attempt)
    return normal((T, H), 1.0, g, device)


def draw_x_rejecting(seed, T, H, accept, device="cpu", tag="x", max_attempts=64):
    """Draw x token by token: token t keeps the row of the first attempt a for
    which accept(rows)[t] is true.  `accept` maps an fp32 [T][H] CPU tensor to
    a bool numpy array [T]; the caller supplies it (the generator holds no
    layer arithmetic).  Returns (x, attempts_per_token)."""
    x = draw_x(seed, T, H, device, tag, 0)
    ok = np.asarray(accept(x.cpu()), dtype=bool)
    att = np.zeros(T, dtype=np.int64)
    a = 0
    while not ok.all():
        a += 1
        if a >= max_attempts:
            raise RuntimeError("rejection sampling did not converge")
        xa = draw_x(seed, T, H, device, tag, a)
        bad = np.nonzero(~ok)[0]
        bad_t = torch.as_tensor(bad, device=x.device)
        x[bad_t] = xa[bad_t]
        att[bad] = a
        ok = np.asarray(accept(x.cpu()), dtype=bool)
    return x, att


def draw_router(seed, layer, E, H, device="cpu"):
    """Router weights as bf16 bits int16 [E][H]."""
    g = make_gen(device, seed, "router", layer)
    return to_bf16_bits(normal((E, H), 0.05, g, device))


def zipf_bias(seed, layer, E, s=1.1):
    """fp32 [E]: b_e = ln p_e, p_e = rank_e^-s / sum_r r^-s."""
    rng = np.random.default_rng(seed_of(seed, "zipf", layer))
    rank = rng.permutation(E) + 1
    p = rank.astype(np.float64) ** (-s)
    p /= p.sum()
    return torch.from_numpy(np.log(p).astype(np.float32))


# ----------------------------------------------------------------------------
# quantisers (weights arrive quantised; these only build inputs)

def quantize_int4(W):
    """W fp32 [..., rows, K] -> (q int8 [..., rows, K] in [-8,7], s fp16 [..., rows, K/32])."""
    *lead, K = W.shape
    Wb = W.reshape(*lead, K // 32, 32)
    s = (Wb.abs().amax(-1) / 7.0).to(torch.float16)
    sf = s.float().unsqueeze(-1)
    q = torch.where(sf > 0, torch.round(Wb / torch.where(sf > 0, sf, torch.ones_like(sf))),
                    torch.zeros_like(Wb))
    q = q.clamp(-8, 7).to(torch.int8).reshape(*lead, K)
    return q, s


def quantize_int2(W):
    """W fp32 [..., rows, K] -> (q uint8 [..., rows, K] in [0,3], s fp16, m fp16 [..., rows, K/16])."""
    *lead, K = W.shape
    Wb = W.reshape(*lead, K // 16, 16)
    lo = Wb.amin(-1)
    hi = Wb.amax(-1)
    m = lo.to(torch.float16)
    s = ((hi - lo) / 3.0).to(torch.float16)
    sf = s.float().unsqueeze(-1)
    q = torch.where(sf > 0,
                    torch.round((Wb - m.float().unsqueeze(-1)) / torch.where(sf > 0, sf, torch.ones_like(sf))),
                    torch.zeros_like(Wb))
    q = q.clamp(0, 3).to(torch.uint8).reshape(*lead, K)
    return q, s, m


# ----------------------------------------------------------------------------
# packers (byte layout of include/moe.h)

def _gu_rows(G, U):
    """[..., F, H] gate/up -> [..., 2F, H] in runs of 32 rows: gate 32, up 32."""
    *lead, F, H = G.shape
    g = G.reshape(*lead, F // 32, 32, H)
    u = U.reshape(*lead, F // 32, 32, H)
    return torch.stack([g, u], dim=-3).reshape(*lead, 2 * F, H)


def _nibble_words(n):
    """n int [..., K] (values 0..15) -> int64 words [..., K/8]:
    word j holds values 8j+2i at bits 4i and 8j+2i+1 at bits 16+4i."""
    *lead, K = n.shape
    v = n.reshape(*lead, K // 8, 4, 2).to(torch.int64)
    sh = torch.arange(4, device=n.device, dtype=torch.int64) * 4
    return (v[..., 0] << sh).sum(-1) | (v[..., 1] << (sh + 16)).sum(-1)


def _crumb_words(n):
    """n [..., K] (values 0..3) -> int64 words [..., K/16]: value 2i at bits 2i
    and value 2i+1 at bits 16+2i."""
    *lead, K = n.shape
    v = n.reshape(*lead, K // 16, 8, 2).to(torch.int64)
    sh = torch.arange(8, device=n.device, dtype=torch.int64) * 2
    return (v[..., 0] << sh).sum(-1) | (v[..., 1] << (sh + 16)).sum(-1)


def _words_to_bytes(w):
    """int64 words holding uint32 values [n, ...] -> uint8 little-endian [n, bytes]."""
    n = w.shape[0]
    w = torch.where(w >= (1 << 31), w - (1 << 32), w)  # uint32 bit pattern as int32
    return w.to(torch.int32).contiguous().view(torch.uint8).reshape(n, -1)


def _f16_bytes(h):
    n = h.shape[0]
    return h.contiguous().view(torch.uint8).reshape(n, -1)


def pack_int4(Wg_q, Wg_s, Wu_q, Wu_s, Wd_q, Wd_s):
    """Quantised int4 matrices of n experts ([n, ...], or one expert without
    the leading n) -> record bytes uint8 [n, R] (resp. [R])."""
    single = Wg_q.dim() == 2
    if single:
        Wg_q, Wg_s, Wu_q, Wu_s, Wd_q, Wd_s = (t.unsqueeze(0) for t in (Wg_q, Wg_s, Wu_q, Wu_s, Wd_q, Wd_s))
    n, F, H = Wg_q.shape
    gu_q = _gu_rows(Wg_q, Wu_q)                                    # [n][2F][H]
    gu_s = _gu_rows(Wg_s, Wu_s)                                    # [n][2F][H/32]
    KBg, KBd = H // 32, F // 32
    wgu = _nibble_words(gu_q.to(torch.int32) + 8).reshape(n, 2 * F, KBg, 4).permute(0, 2, 1, 3)  # [n][kb][r][4]
    wd = _nibble_words(Wd_q.to(torch.int32) + 8).reshape(n, H, KBd, 4).permute(0, 2, 1, 3)
    sgu = gu_s.reshape(n, 2 * F, KBg // 4, 4).permute(0, 2, 1, 3)  # [n][kb/4][r][4]
    sd = Wd_s.permute(0, 2, 1)                                     # [n][kb][r]
    out = torch.cat([_words_to_bytes(wgu), _words_to_bytes(wd), _f16_bytes(sgu), _f16_bytes(sd)], dim=1)
    assert out.shape[1] == record_bytes(QFMT_INT4, H, F)
    return out[0] if single else out


def pack_int2(Wg_q, Wg_s, Wg_m, Wu_q, Wu_s, Wu_m, Wd_q, Wd_s, Wd_m):
    """Quantised int2 matrices of n experts -> record bytes uint8 [n, R] (or [R])."""
    single = Wg_q.dim() == 2
    ts = (Wg_q, Wg_s, Wg_m, Wu_q, Wu_s, Wu_m, Wd_q, Wd_s, Wd_m)
    if single:
        ts = tuple(t.unsqueeze(0) for t in ts)
    Wg_q, Wg_s, Wg_m, Wu_q, Wu_s, Wu_m, Wd_q, Wd_s, Wd_m = ts
    n, F, H = Wg_q.shape
    gu_q = _gu_rows(Wg_q, Wu_q)
    gu_s = _gu_rows(Wg_s, Wu_s)
    gu_m = _gu_rows(Wg_m, Wu_m)
    Ug = H // 64
    wgu = _crumb_words(gu_q.to(torch.int32)).reshape(n, 2 * F, Ug, 4).permute(0, 2, 1, 3)
    wd = _crumb_words(Wd_q.to(torch.int32)).permute(0, 2, 1)        # [n][blk][r]
    mgu = torch.stack([gu_s, gu_m], dim=-1).reshape(n, 2 * F, Ug, 4, 2).permute(0, 2, 1, 3, 4)
    md = torch.stack([Wd_s, Wd_m], dim=-1).permute(0, 2, 1, 3)      # [n][blk][r][2]
    out = torch.cat([_words_to_bytes(wgu), _words_to_bytes(wd), _f16_bytes(mgu), _f16_bytes(md)], dim=1)
    assert out.shape[1] == record_bytes(QFMT_INT2, H, F)
    return out[0] if single else out


def pack_record(qfmt, Wg, Wu, Wd):
    """fp32 weights of one expert ([F][H], [F][H], [H][F]) or of n experts
    (leading dim n) -> record bytes."""
    if qfmt == QFMT_INT4:
        return pack_int4(*quantize_int4(Wg), *quantize_int4(Wu), *quantize_int4(Wd))
    return pack_int2(*quantize_int2(Wg), *quantize_int2(Wu), *quantize_int2(Wd))


def draw_expert_chunks(seed, layer, n_experts, H, F, device="cpu", std=0.02):
    """Yield (e0, Wg [n,F,H], Wu [n,F,H], Wd [n,H,F]) for the experts of one
    layer, EXPERT_CHUNK at a time from one generator per layer (the last
    expert, index E, is the layer's shared expert when n_experts = E+1)."""
    g = make_gen(device, seed, "experts", layer)
    for c0 in range(0, n_experts, EXPERT_CHUNK):
        n = min(EXPERT_CHUNK, n_experts - c0)
        Wg = normal((n, F, H), std, g, device)
        Wu = normal((n, F, H), std, g, device)
        Wd = normal((n, H, F), std, g, device)
        yield c0, Wg, Wu, Wd


def draw_expert_weights(seed, layer, n_experts, H, F, device="cpu", std=0.02):
    """Yield (e, Wg, Wu, Wd) per expert (same draws as draw_expert_chunks)."""
    for c0, Wg, Wu, Wd in draw_expert_chunks(seed, layer, n_experts, H, F, device, std):
        for i in range(Wg.shape[0]):
            yield c0 + i, Wg[i], Wu[i], Wd[i]


def make_slot_table(seed, L, E, n_slots=None):
    """int32 [L][E+1]: a seeded permutation of the L*(E+1) slots."""
    n = L * (E + 1)
    rng = np.random.default_rng(seed_of(seed, "slots"))
    perm = rng.permutation(n if n_slots is None else n_slots)[:n]
    return torch.from_numpy(perm.astype(np.int32).reshape(L, E + 1))


def build_pool(seed, L, E, H, F, qfmt, device="cpu", rec_bytes=None,
               slot_table=None, std=0.02, progress=None):
    """Draw and pack all L*(E+1) records.  Returns (pool uint8 [n*R], S, R)."""
    R = record_bytes(qfmt, H, F) if rec_bytes is None else rec_bytes
    S = make_slot_table(seed, L, E) if slot_table is None else slot_table
    n_slots = int(S.max().item()) + 1
    pool = torch.zeros(n_slots * R, dtype=torch.uint8, device=device)
    view = pool.view(n_slots, R)
    Rq = record_bytes(qfmt, H, F)
    for l in range(L):
        for c0, Wg, Wu, Wd in draw_expert_chunks(seed, l, E + 1, H, F, device, std):
            recs = pack_record(qfmt, Wg, Wu, Wd)                      # [n][Rq]
            slots = S[l, c0:c0 + recs.shape[0]].to(device=device, dtype=torch.long)
            view[slots, :Rq] = recs
            del Wg, Wu, Wd, recs
        if progress is not None:
            progress(l)
    return pool, S, R


def _random_f16(gen, n, lo, hi, p_zero, device):
    """n fp16 values: 0 with probability p_zero, else +-U(lo, hi) (random sign)."""
    mag = torch.rand(n, generator=gen, device=device) * (hi - lo) + lo
    sign = torch.where(torch.rand(n, generator=gen, device=device) < 0.5, -1.0, 1.0)
    zero = torch.rand(n, generator=gen, device=device) < p_zero
    return torch.where(zero, torch.zeros_like(mag), mag * sign).to(torch.float16)


def random_records(gen, qfmt, H, F, n, device="cpu"):
    """n records of uniformly random quantised bytes (every nibble / crumb
    value equally likely, so q = -8 and the int2 range ends occur), with
    random fp16 scales: one in 16 exactly zero, the rest +-U(0.002, 0.008)
    (int4) or +-U(0.004, 0.016) (int2, with mins +-U(0, 0.02), one in 16 zero).
    The meta planes are the records' last bytes (include/moe.h): int4 scales
    from 3HF/2 on, int2 (scale, min) pairs from 3HF/4 on."""
    R = record_bytes(qfmt, H, F)
    recs = torch.randint(0, 256, (n, R), generator=gen, device=device, dtype=torch.int32).to(torch.uint8)
    HF = H * F
    if qfmt == QFMT_INT4:
        m0 = 3 * HF // 2
        nm = (R - m0) // 2
        meta = _random_f16(gen, n * nm, 0.002, 0.008, 1 / 16, device).reshape(n, nm)
    else:
        m0 = 3 * HF // 4
        npair = (R - m0) // 4
        sc = _random_f16(gen, n * npair, 0.004, 0.016, 1 / 16, device).reshape(n, npair)
        mn = _random_f16(gen, n * npair, 0.0, 0.02, 1 / 16, device).reshape(n, npair)
        meta = torch.stack([sc, mn], dim=-1).reshape(n, 2 * npair)
    recs[:, m0:] = meta.contiguous().view(torch.uint8).reshape(n, -1)
    return recs


def build_random_pool(seed, L, E, H, F, qfmt, device="cpu", slot_table=None):
    """A pool of random records (random_records) for all L*(E+1) experts.
    Returns (pool uint8 [n*R], S, R)."""
    R = record_bytes(qfmt, H, F)
    S = make_slot_table(seed, L, E) if slot_table is None else slot_table
    n_slots = int(S.max().item()) + 1
    pool = torch.zeros(n_slots * R, dtype=torch.uint8, device=device)
    view = pool.view(n_slots, R)
    g = make_gen(device, seed, "random-records")
    for l in range(L):
        for c0 in range(0, E + 1, EXPERT_CHUNK):
            nn = min(EXPERT_CHUNK, E + 1 - c0)
            slots = S[l, c0:c0 + nn].to(device=device, dtype=torch.long)
            view[slots] = random_records(g, qfmt, H, F, nn, device)
    return pool, S, R


class LayerInputs:
    """Everything one layer (or a stack) needs, as torch tensors."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def make_layer_inputs(seed, L, E, H, F, qfmt=QFMT_INT4, bias=False,
                      device="cpu", progress=None, hot_slots=0, random_bytes=False):
    """Routers [L][E][H] (bf16 bits), bias [L][E] or None, pool, slot table.
    hot_slots > 0 leaves that many empty record slots at the start of the
    pool (a hot tier); the slot table then holds the home slots after them.
    random_bytes: the records are random_records instead of quantised
    N(0, 0.02) weights."""
    Wr = torch.stack([draw_router(seed, l, E, H, device) for l in range(L)])
    b = torch.stack([zipf_bias(seed, l, E) for l in range(L)]).to(device) if bias else None
    S0 = make_slot_table(seed, L, E) + hot_slots if hot_slots else None
    if random_bytes:
        pool, S, R = build_random_pool(seed, L, E, H, F, qfmt, device, slot_table=S0)
    else:
        pool, S, R = build_pool(seed, L, E, H, F, qfmt, device, slot_table=S0, progress=progress)
    return LayerInputs(seed=seed, L=L, E=E, H=H, F=F, qfmt=qfmt, Wr=Wr, bias=b,
                       pool=pool, S=S.to(device), R=R)
