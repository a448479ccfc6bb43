"""GPU parity of every entry point against the CPU oracle, through the C ABI.

Bars: routing indices, counts, offsets, permutation rows and usage scores /
re-rank bit-exact; routing weights |dw| <= 2e-5 (fp32 sums of 2,048 products
round a logit of size ~2.3 by at most ~1e-5, and a softmax weight moves by at
most twice the largest logit error); MoE outputs rel-L2 <= 2e-3 and max-abs <=
1e-2 * max|y|.  Inputs are seeded (gen/); sizes span several tiles, ragged
tails and empty expert groups, plus the full-size shapes.
"""
import numpy as np
import pytest
import torch

import gen as G
import oracle as O
from tests import cases as C

pytestmark = pytest.mark.gpu

W_ATOL = 2e-5


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_ffn_moe_amd as M
    M.load(build_if_missing=False)
    return M


def _np(t):
    return t.detach().cpu().numpy()


def _check_routing(idx_gpu, w_gpu, idx_ref, w_ref):
    assert np.array_equal(_np(idx_gpu).astype(np.int64), idx_ref)
    assert np.max(np.abs(_np(w_gpu) - w_ref)) <= W_ATOL
    assert np.max(np.abs(_np(w_gpu).sum(1) - 1.0)) <= 1e-6


# ---------------------------------------------------------------- router / top-k

@pytest.mark.parametrize("T,E,k,bias,bf16,H", [(4, 16, 2, False, False, 256), (4, 16, 2, True, True, 256),
                                              (67, 16, 2, False, False, 256), (200, 37, 5, True, True, 256),
                                              (3, 1000, 16, False, False, 256), (5, 16, 16, False, False, 256),
                                              # bf16 chunks on the matrix cores: ragged 128-token and
                                              # 128-expert tiles, E > 512 (16 keys per lane in top-k)
                                              (200, 37, 5, True, True, 384), (300, 512, 10, True, True, 2048),
                                              (33, 40, 6, False, True, 512), (9, 600, 8, True, True, 256)])
def test_route_topk_small(moe, T, E, k, bias, bf16, H):
    Wr = G.draw_router(0, 0, E, H)
    b = G.zipf_bias(0, 0, E) if bias else None
    x, _ = G.draw_x_rejecting(0, T, H, C.gap_acceptor(Wr, b, k, as_bf16=bf16))
    if bf16:
        x = x.to(torch.bfloat16)
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx, w = moe.moe_route_topk(x.cuda(), Wr.cuda(), None if b is None else b.cuda(), k, logits_out=logits)
    ref_l = O.router_logits(C.x_as_f64(x), C.router_f64(Wr), None if b is None else b.double().numpy())
    ref_i, ref_w = O.topk_select(ref_l, k)
    _check_routing(idx, w, ref_i, ref_w)
    assert np.max(np.abs(_np(logits) - ref_l)) <= 1e-4


def test_route_topk_ties_and_zero_router(moe):
    H, E, k, T = 128, 64, 6, 5
    Wr = torch.zeros((E, H), dtype=torch.bfloat16)
    idx, w = moe.moe_route_topk(torch.ones((T, H), device="cuda"), Wr.cuda(), None, k)
    assert _np(idx).tolist() == [list(range(k))] * T
    assert np.all(_np(w) == np.float32(1.0 / k))
    # duplicated rows: equal logits, lower index first
    Wr = G.draw_router(9, 0, E, H)
    Wr[40] = Wr[7]
    Wr[50] = Wr[7]
    x = Wr[7].view(torch.bfloat16).float().unsqueeze(0).repeat(T, 1) * 3.0  # row 7 wins
    idx, w = moe.moe_route_topk(x.cuda(), Wr.cuda(), None, k)
    assert np.all(_np(idx)[:, :3] == [7, 40, 50])
    assert np.all(_np(w)[:, 0] == _np(w)[:, 1])


@pytest.mark.parametrize("T", [1, 4, 8])
def test_route_topk_full_decode(moe, T):
    li_Wr = G.draw_router(1, 0, 512, 2048)
    b = G.zipf_bias(1, 0, 512)
    x, _ = G.draw_x_rejecting(1, T, 2048, C.gap_acceptor(li_Wr, b, 10))
    idx, w = moe.moe_route_topk(x.cuda(), li_Wr.cuda(), b.cuda(), 10)
    ref_i, ref_w = O.topk_select(O.router_logits(C.x_as_f64(x), C.router_f64(li_Wr), b.double().numpy()), 10)
    _check_routing(idx, w, ref_i, ref_w)


def test_route_topk_full_prefill(moe):
    """8,192 bf16 tokens, 512 experts, top-10, no bias (near-uniform routing)."""
    T, H, E, k = 8192, 2048, 512, 10
    Wr = G.draw_router(3, 0, E, H)
    x, att = G.draw_x_rejecting(3, T, H, C.gap_acceptor(Wr, None, k, as_bf16=True))
    x = x.to(torch.bfloat16)
    idx, w = moe.moe_route_topk(x.cuda(), Wr.cuda(), None, k)
    ref_i, ref_w = O.topk_select(O.router_logits(C.x_as_f64(x), C.router_f64(Wr)), k)
    _check_routing(idx, w, ref_i, ref_w)
    counts = np.bincount(ref_i.ravel(), minlength=E)
    assert counts.min() > 0  # a chunk routes to every expert


# ---------------------------------------------------------------- permutation

def _random_idx(rng, T, k, E, skew=0.0):
    p = np.arange(1, E + 1, dtype=np.float64) ** (-skew)
    p /= p.sum()
    return np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,k,E,skew", [(1, 1, 1, 0), (7, 2, 5, 0), (300, 4, 16, 1.5), (1025, 3, 9, 0),
                                        (8192, 10, 512, 0), (16384, 10, 512, 1.1), (50, 16, 1000, 0)])
def test_permute(moe, T, k, E, skew):
    rng = np.random.default_rng(T * 31 + k)
    idx = _random_idx(rng, T, k, E, skew)
    x = torch.randn((T, 64), generator=torch.Generator().manual_seed(T)).to(torch.bfloat16)
    counts, offsets, row_src, inv_row, xp = moe.moe_permute(torch.from_numpy(idx).cuda(), E, x=x.cuda())
    rc, ro, rs, ri = O.permute(idx, E)
    assert np.array_equal(_np(counts), rc)
    assert np.array_equal(_np(offsets), ro)
    assert np.array_equal(_np(row_src), rs)
    assert np.array_equal(_np(inv_row), ri)
    assert torch.equal(xp.cpu(), x[torch.from_numpy(rs) // k])


def test_permute_empty(moe):
    idx = torch.zeros((0, 3), dtype=torch.int32, device="cuda")
    counts, offsets, *_ = moe.moe_permute(idx, 7)
    assert _np(counts).tolist() == [0] * 7 and _np(offsets).tolist() == [0] * 8


@pytest.mark.parametrize("k", list(range(1, 17)))
def test_combine_every_k(moe, k):
    """Both row layouts (prefill: permuted rows + shared; decode: T x (k+1)
    rows) for every k, H not a multiple of 1,024 (a partial workgroup), and
    the residual given as the output buffer itself (the decode chain's use)."""
    T, H = 7, 1028
    g = torch.Generator().manual_seed(100 + k)
    w = torch.rand((T, k), generator=g)
    w = (w / w.sum(1, keepdim=True)).float()
    routed = torch.randn((T, k, H), generator=g)
    shared = torch.randn((T, H), generator=g)
    resid = torch.randn((T, H), generator=g)
    ref = O.combine(routed.double().numpy(), w.double().numpy(), shared.double().numpy(), resid.double().numpy())
    perm = torch.randperm(T * k, generator=g)
    y_perm = torch.empty((T * k, H))
    y_perm[perm] = routed.reshape(T * k, H)
    inv_row = perm.to(torch.int32).reshape(T, k)
    out = resid.clone().cuda()
    moe.moe_combine(y_perm.cuda(), w.cuda(), inv_row=inv_row.cuda(), y_shared=shared.cuda(), residual=out, y_out=out)
    tol = 1e-5 * (np.abs(ref).max() + 1)
    assert np.max(np.abs(_np(out) - ref)) <= tol
    rows = torch.cat([routed, shared.unsqueeze(1)], 1).reshape(T * (k + 1), H)
    y = moe.moe_combine(rows.cuda(), w.cuda(), residual=resid.cuda())
    assert torch.equal(y.cpu(), out.cpu())  # same sums in the same order
    # fp16 rows: the same sums as over their exact fp32 values
    y16 = moe.moe_combine(y_perm.half().cuda(), w.cuda(), inv_row=inv_row.cuda(), y_shared=shared.half().cuda(),
                          residual=resid.cuda())
    y32 = moe.moe_combine(y_perm.half().float().cuda(), w.cuda(), inv_row=inv_row.cuda(),
                          y_shared=shared.half().float().cuda(), residual=resid.cuda())
    assert torch.equal(y16, y32)


# ---------------------------------------------------------------- decode experts

def _layer_outputs_decode(moe, li, x, layer=0):
    idx, w = moe.moe_route_topk(x.cuda(), li.Wr[layer].cuda().contiguous(),
                                None if li.bias is None else li.bias[layer].cuda().contiguous(), li.k)
    yp = moe.moe_expert_gemv_q(x.cuda(), idx, li.E, li.F, li.S.cuda(), layer, li.pool.cuda(), li.R, li.qfmt)
    y = moe.moe_combine(yp, w)
    return idx, w, yp, y


@pytest.mark.parametrize("qfmt", [0, 1])
@pytest.mark.parametrize("T", [1, 4])
def test_gemv_tiny(moe, qfmt, T):
    li = C.layer_case(0, T, 256, 16, 2, 128, qfmt=qfmt)
    idx, w, yp, y = _layer_outputs_decode(moe, li, li.x)
    ry, ri, rw, rparts, _ = C.oracle_layer(li)
    _check_routing(idx, w, ri, rw)
    C.assert_close_moe(_np(yp), rparts, "y_parts")
    C.assert_close_moe(_np(y), ry, "y")


@pytest.mark.parametrize("qfmt", [0, 1])
@pytest.mark.parametrize("T", [1, 4])
def test_gemv_full_layer(moe, qfmt, T):
    """One 512-expert top-10 layer at H=2048, F=768 with the Zipf bias."""
    li = C.layer_case(1, T, 2048, 512, 10, 768, qfmt=qfmt, bias=True, device="cuda")
    idx, w, yp, y = _layer_outputs_decode(moe, li, li.x)
    ry, ri, rw, rparts, _ = C.oracle_layer(li)
    _check_routing(idx, w, ri, rw)
    C.assert_close_moe(_np(yp), rparts, "y_parts")
    C.assert_close_moe(_np(y), ry, "y")


def test_gemv_batch_invariance_and_determinism(moe):
    li = C.layer_case(1, 4, 2048, 512, 10, 768, bias=True, device="cuda")
    _, _, yp4, y4 = _layer_outputs_decode(moe, li, li.x)
    _, _, yp4b, y4b = _layer_outputs_decode(moe, li, li.x)
    assert torch.equal(y4, y4b)  # bit-identical rerun
    for t in range(4):
        idx1, _, yp1, y1 = _layer_outputs_decode(moe, li, li.x[t:t + 1])
        assert torch.equal(yp1[0], yp4[t])  # a token's result does not depend on its batch
        assert torch.equal(y1[0], y4[t])


def test_gemv_slot_permutation_invariance(moe):
    li = C.layer_case(0, 4, 256, 16, 2, 128)
    _, _, _, y = _layer_outputs_decode(moe, li, li.x)
    # move every record to another slot and permute the slot table alike
    n = li.S.numel()
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(5))
    pool2 = torch.zeros_like(li.pool)
    S2 = torch.empty_like(li.S)
    for l in range(li.S.shape[0]):
        for e in range(li.S.shape[1]):
            s_old, s_new = int(li.S[l, e]), int(perm[int(li.S[l, e])])
            pool2[s_new * li.R:(s_new + 1) * li.R] = li.pool[s_old * li.R:(s_old + 1) * li.R]
            S2[l, e] = s_new
    li2 = C.layer_case(0, 4, 256, 16, 2, 128)
    li2.pool, li2.S = pool2, S2
    _, _, _, y2 = _layer_outputs_decode(moe, li2, li.x)
    assert torch.equal(y, y2)


# ---------------------------------------------------------------- prefill experts

def _prefill_layer(moe, li, x_bf16, y_dtype=torch.float16):
    idx, w = moe.moe_route_topk(x_bf16.cuda(), li.Wr[0].cuda().contiguous(),
                                None if li.bias is None else li.bias[0].cuda().contiguous(), li.k)
    counts, offsets, row_src, inv_row, _ = moe.moe_permute(idx, li.E)
    y_perm, y_sh = moe.moe_grouped_gemm_q(x_bf16.cuda(), row_src, offsets, li.k, li.E, li.F, li.S.cuda(), 0,
                                          li.pool.cuda(), li.R, li.qfmt, y_dtype=y_dtype)
    y = moe.moe_combine(y_perm, w, inv_row=inv_row, y_shared=y_sh)
    return idx, w, counts, inv_row, y_perm, y_sh, y


@pytest.mark.parametrize("qfmt", [0, 1])
@pytest.mark.parametrize("T,E,k,bias,H", [(4, 16, 2, False, 256), (300, 16, 2, True, 256), (2000, 16, 2, False, 256),
                                          (333, 40, 6, True, 256), (600, 16, 2, True, 384)])
def test_grouped_gemm_small(moe, qfmt, T, E, k, bias, H):
    """Both output dtypes against the oracle; the fp16 rows are the fp32 rows
    rounded to nearest even, bit for bit (same sums, one rounding).  H = 384:
    the down pass's last 256-column tile has 128 columns, so half of its
    waves have no columns and only help stage the token rows."""
    li = C.layer_case(2, T, H, E, k, 128, qfmt=qfmt, bias=bias, x_bf16=True)
    ry, ri, rw, rparts, _ = C.oracle_layer(li)
    out = {}
    for yd in (torch.float16, torch.float32):
        idx, w, counts, inv_row, y_perm, y_sh, y = _prefill_layer(moe, li, li.x, y_dtype=yd)
        assert y_perm.dtype == yd and y_sh.dtype == yd
        _check_routing(idx, w, ri, rw)
        rows = _np(y_perm)[_np(inv_row).reshape(T, k)]
        C.assert_close_moe(rows, rparts[:, :k], f"routed rows ({yd})")
        C.assert_close_moe(_np(y_sh), rparts[:, k], f"shared ({yd})")
        C.assert_close_moe(_np(y), ry, f"y ({yd})")
        out[yd] = (y_perm, y_sh)
    assert torch.equal(out[torch.float16][0], out[torch.float32][0].half())
    assert torch.equal(out[torch.float16][1], out[torch.float32][1].half())


def test_grouped_gemm_empty_groups(moe):
    """Experts 3, 7 and 11 get no rows; expert 0 gets more than two tiles."""
    T, H, E, k, F = 300, 256, 16, 2, 128
    li = C.layer_case(4, T, H, E, k, F, x_bf16=True, gap=False)
    rng = np.random.default_rng(4)
    pool_e = [e for e in range(1, E) if e not in (3, 7, 11)]
    idx = np.stack([[0, rng.choice(pool_e)] for _ in range(T)]).astype(np.int32)
    counts, offsets, row_src, inv_row, _ = moe.moe_permute(torch.from_numpy(idx).cuda(), E)
    assert _np(counts)[[3, 7, 11]].tolist() == [0, 0, 0]
    y_perm, y_sh = moe.moe_grouped_gemm_q(li.x.cuda(), row_src, offsets, k, E, F, li.S.cuda(), 0, li.pool.cuda(),
                                          li.R, li.qfmt)
    get = O.expert_getter(C.LazyPool(li.pool), li.S.numpy(), 0, li.qfmt, H, F, li.R)
    xf = C.x_as_f64(li.x)
    for e in (0, 1, 15):
        sel = np.nonzero(idx == e)
        ref = O.expert_ffn(*get(e), xf[sel[0]])
        got = _np(y_perm)[_np(inv_row).reshape(T, k)[sel]]
        C.assert_close_moe(got, ref, f"expert {e}")
    C.assert_close_moe(_np(y_sh), O.expert_ffn(*get(E), xf), "shared")


def test_grouped_gemm_full_size_sampled(moe):
    """8,192-token chunk, 512 experts top-10, H=2048, F=768: routing and
    permutation exact on every token, outputs checked on sampled tokens."""
    T, H, E, k, F = 8192, 2048, 512, 10, 768
    li = C.layer_case(3, T, H, E, k, F, x_bf16=True, device="cuda")
    idx, w, counts, inv_row, y_perm, y_sh, y = _prefill_layer(moe, li, li.x)
    xf = C.x_as_f64(li.x)
    ref_i, ref_w = O.topk_select(O.router_logits(xf, C.router_f64(li.Wr[0])), k)
    _check_routing(idx, w, ref_i, ref_w)
    rc, ro, rs, ri = O.permute(ref_i, E)
    assert np.array_equal(_np(counts), rc) and np.array_equal(_np(inv_row), ri)
    sample = np.random.default_rng(0).choice(T, size=12, replace=False)
    sample = np.concatenate([[0, T - 1], sample])
    ry, ri2, rw2, rparts, _ = C.oracle_layer(li, tokens=sample)
    C.assert_close_moe(_np(y)[sample], ry, "y (sampled)")
    rows = _np(y_perm)[_np(inv_row).reshape(T, k)[sample]]
    C.assert_close_moe(rows, rparts[:, :k], "routed rows (sampled)")


def test_grouped_gemm_int2_16k_chunk_sampled(moe):
    """16,384-token chunk through one int2 layer (blocks of 16 with fp16 scale
    and min) under the Zipf routing bias, so expert loads are skewed (about
    320 rows each on average, some far more, possibly none): routing and
    permutation exact on every token, outputs checked on sampled tokens."""
    T, H, E, k, F = 16384, 2048, 512, 10, 768
    li = C.layer_case(4, T, H, E, k, F, qfmt=1, bias=True, x_bf16=True, device="cuda")
    idx, w, counts, inv_row, y_perm, y_sh, y = _prefill_layer(moe, li, li.x)
    xf = C.x_as_f64(li.x)
    b = li.bias[0].cpu().double().numpy()
    ref_i, ref_w = O.topk_select(O.router_logits(xf, C.router_f64(li.Wr[0]), b), k)
    _check_routing(idx, w, ref_i, ref_w)
    rc, ro, rs, ri = O.permute(ref_i, E)
    assert np.array_equal(_np(counts), rc) and np.array_equal(_np(inv_row), ri)
    assert rc.max() > 2 * rc.mean()  # the bias skews the groups
    sample = np.random.default_rng(1).choice(T, size=12, replace=False)
    sample = np.concatenate([[0, T - 1], sample])
    ry, ri2, rw2, rparts, _ = C.oracle_layer(li, tokens=sample)
    C.assert_close_moe(_np(y)[sample], ry, "y (sampled)")
    rows = _np(y_perm)[_np(inv_row).reshape(T, k)[sample]]
    C.assert_close_moe(rows, rparts[:, :k], "routed rows (sampled)")
    C.assert_close_moe(_np(y_sh)[sample], rparts[:, k], "shared (sampled)")


# ---------------------------------------------------------------- usage

def test_usage_update_steps(moe):
    L, E, k, T = 4, 64, 6, 5
    rng = np.random.default_rng(1)
    scores = torch.zeros((L, E), dtype=torch.float32, device="cuda")
    ref = np.zeros((L, E), np.float32)
    hits = torch.empty(E, dtype=torch.int32, device="cuda")
    top = torch.empty(40, dtype=torch.int32, device="cuda")
    for step in range(9):
        for layer in range(L):
            idx = _random_idx(rng, T, k, E, skew=1.2)
            top.fill_(-1)
            moe.moe_usage_update(torch.from_numpy(idx).cuda(), layer, L, E, 0.99, step, 4, 40, hits, scores, top)
            ref, rtop = O.usage_update(ref, idx, layer, 0.99, step, 4, 40)
            assert np.array_equal(_np(scores), ref)  # bit-exact fp32
            if rtop is not None:
                assert np.array_equal(_np(top), rtop)
            else:
                assert np.all(_np(top) == -1)


def test_usage_rerank_full_size(moe):
    L, E = 48, 512
    rng = np.random.default_rng(7)
    s = (rng.integers(0, 50, size=(L, E)) * 0.25).astype(np.float32)  # many ties
    scores = torch.from_numpy(s).cuda()
    hits = torch.empty(E, dtype=torch.int32, device="cuda")
    top = torch.empty(96, dtype=torch.int32, device="cuda")
    idx = _random_idx(rng, 16384, 10, E, skew=1.1)
    moe.moe_usage_update(torch.from_numpy(idx).cuda(), L - 1, L, E, 0.99, 3, 4, 96, hits, scores, top)
    ref, rtop = O.usage_update(s, idx, L - 1, 0.99, 3, 4, 96)
    assert np.array_equal(_np(scores), ref)
    assert np.array_equal(_np(top), rtop)


@pytest.mark.parametrize("T,step", [(1, 3), (4, 7), (4, 2)])
def test_usage_update_stack(moe, T, step):
    """All 48 layers of a step in one launch: bit for bit the oracle's layer
    by layer updates (and its re-rank when the step is a re-rank step), and
    the same as 48 single-layer calls."""
    L, E, k = 48, 512, 10
    rng = np.random.default_rng(40 + T + step)
    s = (rng.integers(0, 50, size=(L, E)) * 0.25).astype(np.float32)
    idx = np.stack([_random_idx(rng, T, k, E, skew=1.1) for _ in range(L)]).astype(np.int32)
    scores = torch.from_numpy(s).cuda()
    hits = torch.empty((L, E), dtype=torch.int32, device="cuda")
    top = torch.full((96,), -1, dtype=torch.int32, device="cuda")
    idx_t = torch.from_numpy(idx).cuda()
    moe.moe_usage_update_stack(idx_t, E, 0.99, step, 4, 96, hits, scores, top)
    ref, rtop = s, None
    for l in range(L):
        ref, t_l = O.usage_update(ref, idx[l], l, 0.99, step, 4, 96)
        rtop = t_l if t_l is not None else rtop
    assert np.array_equal(_np(scores), ref)
    if rtop is not None:
        assert np.array_equal(_np(top), rtop)
    else:
        assert np.all(_np(top) == -1)
    scores2 = torch.from_numpy(s).cuda()
    hits1 = torch.empty(E, dtype=torch.int32, device="cuda")
    top2 = torch.full((96,), -1, dtype=torch.int32, device="cuda")
    for l in range(L):
        moe.moe_usage_update(idx_t[l], l, L, E, 0.99, step, 4, 96, hits1, scores2, top2)
    assert torch.equal(scores2, scores) and torch.equal(top2, top)


# ---------------------------------------------------------------- stacked decode

def _stack_run(moe, li, x, path, ws=None):
    import os
    L, T, H, k = li.Wr.shape[0], x.shape[0], x.shape[1], li.k
    idx_o = torch.empty((L, T, k), dtype=torch.int32, device="cuda")
    w_o = torch.empty((L, T, k), dtype=torch.float32, device="cuda")
    hist = torch.empty((L, T, H), dtype=torch.float32, device="cuda")
    old = os.environ.get("MOE_DECODE_PATH")
    os.environ["MOE_DECODE_PATH"] = path
    try:
        xo = moe.moe_decode_stack(x, li.F, li.E, k, li.Wr, li.bias, li.S, li.pool, li.R, li.qfmt,
                                  topk_idx_out=idx_o, topk_w_out=w_o, x_hist=hist, ws=ws)
    finally:
        if old is None:
            del os.environ["MOE_DECODE_PATH"]
        else:
            os.environ["MOE_DECODE_PATH"] = old
    torch.cuda.synchronize()
    return xo, idx_o, w_o, hist


def _check_stack(li, x, xo, idx_o, w_o, hist, layers):
    """Each listed layer against the oracle fed the kernel's own layer input:
    ids bit-exact, weights within W_ATOL and the layer's output (x_{l+1} - x_l)
    within the MoE tolerance, token by token, for every token whose routing is
    decided by a gap >= MIN_GAP (tokens are independent within a layer, so a
    near tie in one token leaves the others checkable).  Returns (excluded,
    checked) token counts; every token is one or the other."""
    L = hist.shape[0]
    T = hist.shape[1]
    assert torch.equal(hist[0], x)
    assert torch.isfinite(xo).all()
    excluded = checked = 0
    for l in layers:
        xl = torch.from_numpy(O.rms_normalize(C.x_as_f64(hist[l])))
        ry, ri, rw, _, rl = C.oracle_layer(li, layer=l, x=xl)
        ok = O.gap_ok(rl, li.k, C.MIN_GAP)
        excluded += int((~ok).sum())
        checked += int(ok.sum())
        assert np.array_equal(_np(idx_o[l])[ok], ri[ok]), f"layer {l}"
        if ok.any():
            assert np.max(np.abs(_np(w_o[l])[ok] - rw[ok])) <= W_ATOL
        nxt = hist[l + 1] if l + 1 < L else xo
        d = _np(nxt - hist[l])
        for t in np.nonzero(ok)[0]:
            C.assert_close_moe(d[t], ry[t], f"layer {l} token {t}")
    assert excluded + checked == T * len(list(layers))
    return excluded, checked


@pytest.mark.parametrize("path", ["chain", "persistent"])
@pytest.mark.parametrize("qfmt", [0, 1])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 8])
def test_decode_stack_tiny(moe, qfmt, T, path):
    L = 6
    li = C.layer_case(5, T, 256, 16, 2, 128, qfmt=qfmt, bias=True, L=L, gap=False, device="cuda")
    x = li.x.contiguous()
    xo, idx_o, w_o, hist = _stack_run(moe, li, x, path)
    excluded, checked = _check_stack(li, x, xo, idx_o, w_o, hist, range(L))
    assert excluded <= T * L // 4


@pytest.mark.parametrize("qfmt", [0, 1])
@pytest.mark.parametrize("T,k", [(1, 10), (2, 10), (3, 10), (4, 10), (1, 6), (4, 6), (3, 5)])
def test_decode_stack_full_shape_persistent(moe, qfmt, T, k):
    """4 layers of the full shape (512 experts, H=2048, F=768; top-10, and the
    smaller k of a faster routing mode): the persistent kernel and the kernel
    chain, each checked against the oracle on every layer (the oracle fed that
    path's own layer inputs); the two paths agree on layer 0, where their
    inputs are identical."""
    L = 4
    li = C.layer_case(6, T, 2048, 512, k, 768, qfmt=qfmt, bias=True, L=L, gap=False, device="cuda")
    x = li.x.contiguous()
    ws = moe.workspace(moe.MOE_OP_DECODE_STACK, "cuda", T, k, 512, 2048, 768, qfmt)
    xo, idx_o, w_o, hist = _stack_run(moe, li, x, "persistent", ws=ws)
    excluded, _ = _check_stack(li, x, xo, idx_o, w_o, hist, range(L))
    xc, idx_c, w_c, hist_c = _stack_run(moe, li, x, "chain")
    excluded += _check_stack(li, x, xc, idx_c, w_c, hist_c, range(L))[0]
    assert excluded <= 2 * T * L // 4
    # Layer 0: the same input.  The paths sum the router dot products in
    # different orders, so two nearly equal logits may come out in either
    # order; such a swap leaves the weight at every position equal within
    # W_ATOL.  Any other difference in the ids is an error.
    same = (idx_c[0] == idx_o[0]).all(-1)
    w_close = (w_c[0] - w_o[0]).abs().amax(-1) <= W_ATOL
    assert bool((same | w_close).all()), "layer-0 expert ids differ beyond a near-tie swap"
    keep = (idx_c[0].sort(-1).values == idx_o[0].sort(-1).values).all(-1)
    C.assert_close_moe(_np((hist_c[1] - x)[keep]), _np((hist[1] - x)[keep]), "layer 0: chain vs persistent")
    # repeated calls on the same workspace: new tags each call, same result
    for rep in range(3):
        xo2, idx2, _, _ = _stack_run(moe, li, x, "persistent", ws=ws)
        assert torch.equal(xo2, xo) and torch.equal(idx2, idx_o)


@pytest.mark.parametrize("qfmt", [0, 1])
@pytest.mark.parametrize("T,k", [(5, 10), (6, 10), (8, 10), (6, 6), (8, 8)])
def test_decode_stack_wide_verify(moe, qfmt, T, k):
    """Verify windows of 5, 6 and 8 token positions, 4 layers of the full
    shape: the default path (the persistent kernel) and the per-layer kernel
    chain, each layer checked against the
    oracle on the path's own layer inputs, and the same step repeated bit for
    bit on the same workspace."""
    L = 4
    li = C.layer_case(9, T, 2048, 512, k, 768, qfmt=qfmt, bias=True, L=L, gap=False, device="cuda")
    x = li.x.contiguous()
    ws = moe.workspace(moe.MOE_OP_DECODE_STACK, "cuda", T, k, 512, 2048, 768, qfmt)
    xo, idx_o, w_o, hist = _stack_run(moe, li, x, "auto", ws=ws)
    excluded, _ = _check_stack(li, x, xo, idx_o, w_o, hist, range(L))
    xc, idx_c, w_c, hist_c = _stack_run(moe, li, x, "chain")
    excluded += _check_stack(li, x, xc, idx_c, w_c, hist_c, range(L))[0]
    assert excluded <= 2 * T * L // 4
    for rep in range(2):
        xo2, idx2, _, _ = _stack_run(moe, li, x, "auto", ws=ws)
        assert torch.equal(xo2, xo) and torch.equal(idx2, idx_o)


@pytest.mark.parametrize("qfmt", [0, 1])
def test_decode_stack_48_layers(moe, qfmt):
    """The whole 48-layer stack (int4: 65 GB pool; int2: 58 GB; Zipf routing
    bias), one token, the persistent kernel: every layer input finite, and
    layers 0, 16, 32 and 47 checked against the oracle on the kernel's own
    layer inputs."""
    L = 48
    li = C.layer_case(2, 1, 2048, 512, 10, 768, qfmt=qfmt, bias=True, L=L, device="cuda")
    x = li.x.contiguous()
    xo, idx_o, w_o, hist = _stack_run(moe, li, x, "persistent")
    assert bool(torch.isfinite(hist).all()) and bool(torch.isfinite(xo).all())
    excluded, _ = _check_stack(li, x, xo, idx_o, w_o, hist, [0, 16, 32, 47])
    assert excluded <= 2  # layer 0 is gap-filtered; later layers may hold a near tie


@pytest.mark.parametrize("T", [1, 4])
def test_decode_stack_router_ties(moe, T):
    """A zero router makes every logit equal its bias, so the persistent
    kernel's top-k sees exact ties: all 512 logits equal (more candidates than
    one wave ranks at once), runs of 8 equal values, 64 distinct values each
    held by 8 experts in scattered positions, and 40 values drawn with many
    repeats.  The ids follow the lower-index rule exactly; the weights and
    each layer's output match the oracle."""
    L, E, k = 4, 512, 10
    li = C.layer_case(8, T, 2048, E, k, 768, qfmt=0, bias=True, L=L, gap=False, device="cuda")
    li.Wr = torch.zeros_like(li.Wr)
    rng = np.random.default_rng(3)
    b = np.zeros((L, E), np.float32)
    b[0] = 0.5
    b[1] = -(np.arange(E) // 8) * 0.25
    b[2] = (np.arange(E) * 37 % 64) * 0.125
    b[3] = rng.integers(0, 40, E) * 0.0625
    li.bias = torch.from_numpy(b).cuda()
    x = li.x.contiguous()
    xo, idx_o, w_o, hist = _stack_run(moe, li, x, "persistent")
    assert bool(torch.isfinite(xo).all())
    for l in range(L):
        ri, rw = O.topk_select(np.repeat(b[l][None].astype(np.float64), T, 0), k)
        assert np.array_equal(_np(idx_o[l]), ri), f"layer {l}"
        assert np.max(np.abs(_np(w_o[l]) - rw)) <= W_ATOL
        xl = torch.from_numpy(O.rms_normalize(C.x_as_f64(hist[l])))
        ry = C.oracle_layer(li, layer=l, x=xl)[0]
        nxt = hist[l + 1] if l + 1 < L else xo
        C.assert_close_moe(_np(nxt - hist[l]), ry, f"layer {l}")


# ---------------------------------------------------------------- generator

@pytest.mark.parametrize("qfmt", [0, 1])
def test_packer_on_gpu_is_a_valid_encoding(moe, qfmt):
    """The large pools are packed on the GPU.  Its bytes decode (oracle decoder)
    to within the quantisation step of the drawn weights and match the CPU
    packing except where a value sits on a rounding boundary (the two
    devices' fp32 division may round such w/s differently)."""
    g = G.make_gen("cpu", 77, qfmt)
    Wg, Wu, Wd = (G.normal((3,) + s, 0.02, g, "cpu") for s in [(128, 256), (128, 256), (256, 128)])
    a = G.pack_record(qfmt, Wg, Wu, Wd)
    b = G.pack_record(qfmt, Wg.cuda(), Wu.cuda(), Wd.cuda()).cpu()
    for e in range(3):
        da = O.decode_record(a[e].numpy(), qfmt, 256, 128)
        db = O.decode_record(b[e].numpy(), qfmt, 256, 128)
        for W, A, B in zip((Wg[e], Wu[e], Wd[e]), da, db):
            W = W.double().numpy()
            step = np.abs(A - W).max() * 2 + 1e-12
            assert np.abs(B - W).max() <= step * 1.01
            assert np.mean(A != B) < 1e-3


# ---------------------------------------------------------------- hot tier

from oracle import tier as TI  # noqa: E402


def _tier_case(rng, L, E, n_hot, R):
    """A pool of n_hot hot slots (zeroed) followed by every expert's home
    record (random bytes) at a shuffled home slot."""
    home = (n_hot + rng.permutation(L * (E + 1))).astype(np.int32).reshape(L, E + 1)
    pool = torch.zeros((n_hot + L * (E + 1)) * R, dtype=torch.uint8, device="cuda")
    pool[n_hot * R:] = torch.from_numpy(rng.integers(0, 256, size=L * (E + 1) * R, dtype=np.uint8)).cuda()
    return home, pool


def _tier_state_equal(moe_state, ref, E, check_swaps=True):
    slot, owner, swaps, n_sw = moe_state
    r_slot, r_owner, r_swaps = ref
    assert np.array_equal(_np(slot), r_slot)
    assert np.array_equal(_np(owner), r_owner)
    assert int(n_sw.item()) == len(r_swaps)
    if check_swaps and r_swaps:
        assert np.array_equal(_np(swaps)[:len(r_swaps)], np.array(r_swaps, np.int32))


def _tier_records_ok(pool, slot, home, R, E):
    """Every routed expert's record, read through the slot table, is its home
    record byte for byte."""
    v = pool.view(-1, R)
    s = torch.from_numpy(np.asarray(slot)[:, :E].reshape(-1).astype(np.int64)).cuda()
    h = torch.from_numpy(np.asarray(home)[:, :E].reshape(-1).astype(np.int64)).cuda()
    assert torch.equal(v[s], v[h])


@pytest.mark.parametrize("L,E,n_hot,R", [(3, 16, 12, 4096), (2, 40, 80, 256), (48, 512, 4096, 256)])
def test_tier_fill_and_rebalance(moe, L, E, n_hot, R):
    """The tier's fill and several rebalance rounds (scores with many ties;
    capped, uncapped and empty rounds; a tier that holds every expert) against
    the oracle bit for bit: slot table, hot-slot owners, swap list; every record read through
    the slot table equals its home record."""
    rng = np.random.default_rng(L * 1000 + E)
    home, pool = _tier_case(rng, L, E, n_hot, R)
    home_t = torch.from_numpy(home).cuda()
    slot = torch.empty_like(home_t)
    owner = torch.empty(n_hot, dtype=torch.int32, device="cuda")
    swaps = torch.full((max(n_hot, 1024), 4), -7, dtype=torch.int32, device="cuda")
    n_sw = torch.zeros(1, dtype=torch.int32, device="cuda")
    prof = (rng.integers(0, 40, size=(L, E)) * 0.25).astype(np.float32)
    moe.moe_tier_fill(torch.from_numpy(prof).cuda(), n_hot, home_t, slot, owner, pool, R, swaps, n_sw)
    torch.cuda.synchronize()
    ref = TI.tier_fill(prof, n_hot, home)
    _tier_state_equal((slot, owner, swaps, n_sw), ref, E)
    _tier_records_ok(pool, _np(slot), home, R, E)
    r_slot, r_owner = ref[0], ref[1]
    for cap in [96, 5, 1024, 0, 64, 1, 96]:
        sc = (rng.integers(0, 40, size=(L, E)) * 0.25).astype(np.float32)
        moe.moe_tier_rebalance(torch.from_numpy(sc).cuda(), n_hot, cap, home_t, slot, owner, pool, R, swaps, n_sw)
        torch.cuda.synchronize()
        ref = TI.tier_rebalance(sc, n_hot, cap, home, r_slot, r_owner)
        _tier_state_equal((slot, owner, swaps, n_sw), ref, E)
        r_slot, r_owner = ref[0], ref[1]
        _tier_records_ok(pool, _np(slot), home, R, E)


def test_tier_decode_reads_through_the_tier(moe):
    """A 2-layer decode step through a tiered pool (hot copies after a fill and
    a rebalance) is bit-identical to the same step on the home records."""
    L, T = 2, 2
    li = C.layer_case(5, T, 256, 16, 2, 128, qfmt=0, bias=True, L=L, gap=False, device="cuda")
    n_hot, E, R = 8, 16, li.R
    home_t = (li.S + n_hot).to(torch.int32).contiguous()
    pool = torch.cat([torch.zeros(n_hot * R, dtype=torch.uint8, device="cuda"), li.pool])
    x = li.x.contiguous()
    ref = moe.moe_decode_stack(x, li.F, E, li.k, li.Wr, li.bias, home_t, pool, R, li.qfmt)
    slot = torch.empty_like(home_t)
    owner = torch.empty(n_hot, dtype=torch.int32, device="cuda")
    swaps = torch.empty((1024, 4), dtype=torch.int32, device="cuda")
    n_sw = torch.zeros(1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(4)
    prof = torch.from_numpy(rng.uniform(0, 5, size=(L, E)).astype(np.float32)).cuda()
    moe.moe_tier_fill(prof, n_hot, home_t, slot, owner, pool, R, swaps, n_sw)
    sc = rng.uniform(0, 5, size=(L, E)).astype(np.float32)
    moe.moe_tier_rebalance(torch.from_numpy(sc).cuda(), n_hot, 96, home_t, slot, owner, pool, R, swaps, n_sw)
    torch.cuda.synchronize()
    assert int((slot[:, :E] < n_hot).sum().item()) == n_hot  # the tier is in use
    for path in ("persistent", "chain"):
        import os
        old = os.environ.get("MOE_DECODE_PATH")
        os.environ["MOE_DECODE_PATH"] = path
        try:
            got = moe.moe_decode_stack(x, li.F, E, li.k, li.Wr, li.bias, slot, pool, R, li.qfmt)
            base = moe.moe_decode_stack(x, li.F, E, li.k, li.Wr, li.bias, home_t, pool, R, li.qfmt)
        finally:
            if old is None:
                del os.environ["MOE_DECODE_PATH"]
            else:
                os.environ["MOE_DECODE_PATH"] = old
        torch.cuda.synchronize()
        assert torch.equal(got, base), path
    assert torch.isfinite(ref).all()
