"""Pins of the CPU oracle against things other than itself: hand-derived
fixtures of the byte format, closed forms, brute force on tiny inputs,
identities and library routines.  CPU only."""
import json
import math
import os
import struct

import numpy as np
import pytest
import scipy.special
import torch

import gen as G
import oracle as O
from oracle import tier as T

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _fixture(name):
    with open(os.path.join(GOLD, name)) as f:
        d = json.load(f)
    rec = np.zeros(d["record_bytes"], np.uint8)
    for w in d["writes"]:
        b = np.frombuffer(bytes.fromhex(w["hex"]), np.uint8)
        rec[w["offset"]:w["offset"] + b.size] = b
    return d, rec


# ---------------------------------------------------------------- format

def test_record_sizes():
    # 27HF/16 and 3HF/2 bytes; at H=2048, F=768: 648 and 576 pages of 4 KiB
    assert G.record_bytes(0, 2048, 768) == 2_654_208 == 648 * 4096
    assert G.record_bytes(1, 2048, 768) == 2_359_296 == 576 * 4096
    assert G.record_bytes(0, 256, 128) == 55_296


@pytest.mark.parametrize("name", ["format_int4.json", "format_int2.json"])
def test_decode_hand_made_record(name):
    d, rec = _fixture(name)
    assert rec.size == G.record_bytes(d["qfmt"], d["H"], d["F"])
    Wg, Wu, Wd = O.decode_record(rec, d["qfmt"], d["H"], d["F"])
    assert Wg.shape == (d["F"], d["H"]) and Wu.shape == (d["F"], d["H"]) and Wd.shape == (d["H"], d["F"])
    mats = {"gate": Wg, "up": Wu, "down": Wd}
    listed = {m: np.zeros(M.shape, bool) for m, M in mats.items()}
    for ex in d["expect"]:
        vals = ex["values"] if "values" in ex else [ex["fill"]] * ex["n"]
        got = mats[ex["m"]][ex["row"], ex["col0"]:ex["col0"] + len(vals)]
        np.testing.assert_array_equal(got, np.array(vals, np.float64), err_msg=str(ex))
        listed[ex["m"]][ex["row"], ex["col0"]:ex["col0"] + len(vals)] = True
    for m, M in mats.items():
        assert np.all(M[~listed[m]] == 0), m


@pytest.mark.parametrize("qfmt", [0, 1])
def test_quantise_decode_round_trip(qfmt):
    H, F = 256, 128
    g = G.make_gen("cpu", 123, "rt", qfmt)
    Wg, Wu, Wd = (G.normal(s, 0.02, g, "cpu") for s in [(F, H), (F, H), (H, F)])
    rec = G.pack_record(qfmt, Wg, Wu, Wd).numpy()
    dec = O.decode_record(rec, qfmt, H, F)
    for W, D in zip((Wg, Wu, Wd), dec):
        if qfmt == 0:
            q, s = G.quantize_int4(W)
            blk = 32
            exact = q.double().numpy() * np.repeat(s.double().numpy(), blk, axis=1)
            bound = np.repeat(s.double().numpy(), blk, axis=1) / 2
        else:
            q, s, m = G.quantize_int2(W)
            blk = 16
            sr = np.repeat(s.double().numpy(), blk, axis=1)
            mr = np.repeat(m.double().numpy(), blk, axis=1)
            exact = q.double().numpy() * sr + mr
            lo = W.double().numpy().reshape(W.shape[0], -1, blk).min(-1)
            hi = W.double().numpy().reshape(W.shape[0], -1, blk).max(-1)
            # s/2 plus what the fp16 rounding of m and s moves the grid ends
            slack = np.abs(np.repeat(lo, blk, 1) - mr) + np.abs(3 * sr - np.repeat(hi - lo, blk, 1))
            bound = sr / 2 + slack
        np.testing.assert_array_equal(D, exact)  # decoder == quantiser's (q, s[, m])
        assert np.all(np.abs(W.double().numpy() - D) <= bound * (1 + 1e-6) + 1e-12)


# ---------------------------------------------------------------- router / top-k

def _brute_topk(x, Wr, b, k):
    T, E = len(x), len(Wr)
    idx, w = [], []
    for t in range(T):
        l = [math.fsum(x[t][h] * Wr[e][h] for h in range(len(x[t]))) + (b[e] if b is not None else 0.0)
             for e in range(E)]
        order = sorted(range(E), key=lambda e: (-l[e], e))[:k]
        z = [math.exp(l[e] - l[order[0]]) for e in order]
        idx.append(order)
        w.append([v / math.fsum(z) for v in z])
    return np.array(idx), np.array(w)


def test_topk_brute_force_tiny():
    rng = np.random.default_rng(5)
    for trial in range(20):
        T, E, H = 3, int(rng.integers(2, 9)), 5
        k = int(rng.integers(1, E + 1))
        x = rng.normal(size=(T, H))
        Wr = rng.normal(size=(E, H))
        b = rng.normal(size=E) if trial % 2 else None
        idx, w = O.topk_select(O.router_logits(x, Wr, b), k)
        bi, bw = _brute_topk(x.tolist(), Wr.tolist(), None if b is None else b.tolist(), k)
        np.testing.assert_array_equal(idx, bi)
        np.testing.assert_allclose(w, bw, rtol=0, atol=1e-14)


def test_ties_go_to_lower_index():
    H, E, k = 8, 6, 3
    Wr = np.zeros((E, H))
    Wr[5] = Wr[2] = np.arange(1, H + 1)   # identical best rows 2 and 5
    Wr[4] = 0.5 * np.arange(1, H + 1)
    x = np.ones((1, H))
    idx, w = O.topk_select(O.router_logits(x, Wr), k)
    assert idx.tolist() == [[2, 5, 4]]
    assert w[0, 0] == w[0, 1]


def test_all_zero_router_picks_first_k_uniformly():
    idx, w = O.topk_select(O.router_logits(np.ones((2, 16)), np.zeros((10, 16))), 4)
    assert idx.tolist() == [[0, 1, 2, 3]] * 2
    assert np.all(w == 0.25)


def test_k2_closed_form_and_full_softmax_renormalised():
    rng = np.random.default_rng(1)
    l = rng.normal(size=(50, 12)) * 2
    idx, w = O.topk_select(l, 2)
    l0 = l[np.arange(50), idx[:, 0]]
    l1 = l[np.arange(50), idx[:, 1]]
    np.testing.assert_allclose(w[:, 0], 1.0 / (1.0 + np.exp(l1 - l0)), rtol=1e-14)
    # softmax over all experts, then renormalised over the chosen k
    for k in (1, 3, 7, 12):
        idx, w = O.topk_select(l, k)
        p = scipy.special.softmax(l, axis=1)
        pk = np.take_along_axis(p, idx, 1)
        np.testing.assert_allclose(w, pk / pk.sum(1, keepdims=True), rtol=1e-12)
        assert np.all([len(set(r)) == k for r in idx.tolist()])
        np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)
        assert np.all(np.diff(np.take_along_axis(l, idx, 1), axis=1) <= 0)


def test_gap_helpers():
    l = np.array([[5.0, 4.0, 4.0005, 1.0], [3.0, 2.0, 1.0, 0.0]])
    np.testing.assert_allclose(O.topk_gaps(l, 2), [0.0005, 1.0])
    assert O.gap_ok(l, 2).tolist() == [False, True]
    assert O.gap_ok(l, 1).tolist() == [True, True]


# ---------------------------------------------------------------- experts

def test_silu_identities_and_library():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(O.silu(z) - O.silu(-z), z, rtol=0, atol=1e-12)
    assert O.silu(0.0) == 0.0
    assert abs(O.silu(60.0) - 60.0) < 1e-20 and abs(O.silu(-60.0)) < 1e-20
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    np.testing.assert_allclose(O.silu(z), ref, rtol=1e-15, atol=1e-300)


def test_swiglu_hand_example():
    # Wg = I, Wu = 2I, Wd = I, x = (ln3, -ln3, 0):
    # silu(ln3) = ln3 * 3/4, silu(-ln3) = -ln3 / 4, so y = (1.5 ln^2 3, 0.5 ln^2 3, 0)
    L3 = math.log(3.0)
    I = np.eye(3)
    y = O.expert_ffn(I, 2 * I, I, np.array([[L3, -L3, 0.0]]))
    np.testing.assert_allclose(y[0], [1.5 * L3 * L3, 0.5 * L3 * L3, 0.0], rtol=1e-15, atol=1e-300)


def test_expert_operand_orientation():
    # rectangular shapes: Wg, Wu are [F][H], Wd is [H][F]
    H, F = 4, 2
    Wg = np.zeros((F, H)); Wg[1, 2] = 1.0      # g1 = x2
    Wu = np.zeros((F, H)); Wu[1, 0] = 1.0      # u1 = x0
    Wd = np.zeros((H, F)); Wd[3, 1] = 5.0      # y3 = 5 h1
    x = np.array([[2.0, 0.0, math.log(3.0), 0.0]])
    y = O.expert_ffn(Wg, Wu, Wd, x)
    np.testing.assert_allclose(y[0], [0, 0, 0, 5 * 0.75 * math.log(3.0) * 2.0], rtol=1e-15)


def _scaled_identity_experts(a, b, H):
    """Expert e: Wg = a_e I, Wu = I, Wd = b_e I, so y_e(x) = b_e silu(a_e x) x."""
    I = np.eye(H)
    return lambda e: (a[e] * I, I, b[e] * I)


def test_dense_mixture_when_k_equals_E():
    rng = np.random.default_rng(7)
    T, H, E = 5, 6, 4
    a = rng.normal(size=E + 1); b = rng.normal(size=E + 1)
    x = rng.normal(size=(T, H)); Wr = rng.normal(size=(E, H))
    y, idx, w, _, l = O.moe_layer(x, Wr, None, E, _scaled_identity_experts(a, b, H), E)
    xt = torch.from_numpy(x)
    p = torch.softmax(torch.from_numpy(x @ Wr.T), dim=1)
    ref = sum(p[:, e:e + 1] * b[e] * torch.nn.functional.silu(a[e] * xt) * xt for e in range(E))
    ref = ref + b[E] * torch.nn.functional.silu(a[E] * xt) * xt
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_single_expert_and_zero_down():
    rng = np.random.default_rng(8)
    T, H = 3, 5
    a = rng.normal(size=2); b = rng.normal(size=2)
    x = rng.normal(size=(T, H))
    get = _scaled_identity_experts(a, b, H)
    y, idx, w, parts, _ = O.moe_layer(x, rng.normal(size=(1, H)), None, 1, get, 1)
    assert np.all(idx == 0) and np.all(w == 1.0)
    np.testing.assert_allclose(y, b[0] * O.silu(a[0] * x) * x + b[1] * O.silu(a[1] * x) * x, rtol=1e-13)
    # routed experts with a zero down matrix leave only the shared expert
    E = 6
    b2 = np.zeros(E + 1); b2[E] = 1.5
    a2 = rng.normal(size=E + 1)
    y, *_ = O.moe_layer(x, rng.normal(size=(E, H)), None, 3, _scaled_identity_experts(a2, b2, H), E)
    np.testing.assert_allclose(y, 1.5 * O.silu(a2[E] * x) * x, rtol=1e-14)


def test_combine_hand_example():
    yr = np.array([[[1.0, 2.0], [10.0, 20.0]]])
    ys = np.array([[100.0, 200.0]])
    w = np.array([[0.25, 0.75]])
    np.testing.assert_array_equal(O.combine(yr, w, ys), [[107.75, 215.5]])
    np.testing.assert_array_equal(O.combine(yr, w, ys, residual=np.array([[1.0, -1.0]])), [[108.75, 214.5]])


# ---------------------------------------------------------------- permutation

def test_permute_brute_force_and_invariants():
    rng = np.random.default_rng(3)
    for T, k, E in [(1, 1, 1), (7, 2, 5), (40, 4, 9), (100, 10, 512), (3, 3, 1000)]:
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
        counts, offsets, row_src, inv_row = O.permute(idx, E)
        flat = idx.reshape(-1).tolist()
        brute = sorted(range(T * k), key=lambda i: (flat[i], i))
        assert row_src.tolist() == brute
        assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
        assert counts.tolist() == [flat.count(e) for e in range(E)]
        assert np.all(inv_row[row_src] == np.arange(T * k))
        X = rng.normal(size=(T, 3))
        xp = X[row_src // k]                                   # permute
        back = xp[inv_row].reshape(T, k, 3)                    # unpermute
        assert np.all(back == X[:, None, :])
        for e in range(E):
            seg = row_src[offsets[e]:offsets[e + 1]]
            assert np.all(idx.reshape(-1)[seg] == e) and np.all(np.diff(seg) > 0)


# ---------------------------------------------------------------- usage

def _r32(v):
    return struct.unpack("f", struct.pack("f", v))[0]


def test_usage_emulates_fp32_one_rounding_per_op():
    rng = np.random.default_rng(11)
    L, E = 3, 20
    s = rng.uniform(0, 50, size=(L, E)).astype(np.float32)
    idx = np.stack([rng.choice(E, 4, replace=False) for _ in range(6)])
    new, top = O.usage_update(s, idx, 1, 0.99, 0, 4, 5)
    hits = [sum(1 for row in idx.tolist() if e in row) for e in range(E)]
    d32 = _r32(0.99)
    for e in range(E):
        assert new[1, e] == _r32(_r32(d32 * float(s[1, e])) + hits[e])
    assert np.array_equal(new[[0, 2]], s[[0, 2]]) and top is None


def test_usage_closed_form_and_rerank():
    L, E, h = 2, 8, 3
    s = np.zeros((L, E), np.float32)
    idx = np.array([[0, 1]] * h)  # experts 0 and 1 get h hits per step
    tops = {}
    for n in range(1, 41):
        for layer in range(L):
            s, top = O.usage_update(s, idx if layer == 0 else idx + 2, layer, 0.99, n - 1, 4, 5)
            if top is not None:
                tops[n] = top
        expect = h * (1 - 0.99 ** n) / 0.01
        assert abs(float(s[0, 0]) - expect) <= 1e-5 * expect
    assert sorted(tops) == list(range(4, 41, 4))
    # ties between equal scores go to the lower flat index: 0,1 (layer 0), 10,11 (layer 1)
    assert tops[40].tolist() == [0, 1, 10, 11, 2]


def test_usage_topn_brute_force():
    rng = np.random.default_rng(2)
    L, E = 4, 30
    s = rng.integers(0, 6, size=(L, E)).astype(np.float32)   # many ties
    new, top = O.usage_update(s, np.zeros((0, 3), np.int64), L - 1, 0.5, 3, 4, 17)
    flat = new.reshape(-1).tolist()
    brute = sorted(range(L * E), key=lambda i: (-flat[i], i))[:17]
    assert top.tolist() == brute


# ---------------------------------------------------------------- hot tier

def _tier_home(L, E, n_hot):
    return np.array([[n_hot + l * (E + 1) + e for e in range(E + 1)] for l in range(L)], np.int32)


def _tier_consistent(slot, owner, home, E):
    """Every hot slot's expert points at that slot, every other expert at its
    home record, no expert held twice, the shared column never touched."""
    held = [int(f) for f in owner if f >= 0]
    assert len(held) == len(set(held))
    L = home.shape[0]
    for f in range(L * E):
        l, e = divmod(f, E)
        want = [i for i, o in enumerate(owner) if o == f]
        want = want[0] if want else None
        if want is not None:
            assert owner[want] == f and slot[l][e] == want
        else:
            assert slot[l][e] == home[l][e]
    assert np.array_equal(np.asarray(slot)[:, E], home[:, E])


def test_tier_worked_example():
    g = json.load(open(os.path.join(GOLD, "tier_small.json")))
    L, E, n = g["L"], g["E"], g["n_hot"]
    home = _tier_home(L, E, n)
    slot, owner, swaps = T.tier_fill(np.array(g["profile"], np.float32), n, home)
    assert owner.tolist() == g["fill_owner"] and slot.tolist() == g["fill_slot_table"]
    assert [sw[2] for sw in swaps] == [0, 1, 2] and all(sw[1] == -1 for sw in swaps)
    start = home.copy()
    for i, f in enumerate(g["owner"]):
        start[f // E][f % E] = i
    sc = np.array(g["scores"], np.float32)
    slot, owner, swaps = T.tier_rebalance(sc, n, g["max_swaps"], home, start, g["owner"])
    assert [list(sw) for sw in swaps] == g["swaps"] and owner.tolist() == g["rebalance_owner"]
    _tier_consistent(slot, owner, home, E)
    swaps3 = T.tier_rebalance(sc, n, 3, home, start, g["owner"])[2]
    assert [list(sw) for sw in swaps3] == g["max_swaps_3_swaps"]
    sc[0][0] = 2.0
    swaps_tie = T.tier_rebalance(sc, n, 3, home, start, g["owner"])[2]
    assert [list(sw) for sw in swaps_tie] == g["tie_swaps"]
    # residents 1 and 2 scored alike: the higher index (2, in slot 1) goes first
    sc2 = np.array(g["scores"], np.float32)
    sc2[0][1] = sc2[0][2] = 1.0
    assert T.tier_rebalance(sc2, n, 1, home, start, g["owner"])[2] == [(6, 2, 1, 10)]
    # empty slots are taken first, the lower slot first: owner [-1, 2, -1]
    part = home.copy()
    part[0][2] = 1
    sw = T.tier_rebalance(np.array(g["scores"], np.float32), n, 3, home, part, [-1, 2, -1])[2]
    assert [(c, v, d) for c, v, d, _ in sw] == [(6, -1, 0), (3, -1, 2), (0, 2, 1)]


@pytest.mark.parametrize("seed", range(6))
def test_tier_fill_and_rebalance_brute_force(seed):
    """Random tiers (ties, empty slots, caps): the fill holds exactly the
    brute-force top n_hot; after a rebalance no expert left outside scores
    strictly above any resident, unless the swap cap stopped it, and the
    swapped-in experts are the best-ranked non-residents, in rank order."""
    rng = np.random.default_rng(100 + seed)
    L, E = int(rng.integers(1, 4)), int(rng.integers(3, 12))
    N = L * E
    n_hot = int(rng.integers(1, N + 1))
    home = _tier_home(L, E, n_hot)
    prof = rng.integers(0, 5, size=(L, E)).astype(np.float32)
    slot, owner, _ = T.tier_fill(prof, n_hot, home)
    key = lambda sc: (lambda i: (-float(sc.reshape(-1)[i]), i))
    assert sorted(owner.tolist()) == sorted(sorted(range(N), key=key(prof))[:n_hot])
    assert owner.tolist() == sorted(owner.tolist())
    _tier_consistent(slot, owner, home, E)
    # start from a random partial tier: some slots empty
    owner = np.full(n_hot, -1, np.int32)
    held = rng.choice(N, size=int(rng.integers(0, n_hot + 1)), replace=False)
    pos = rng.choice(n_hot, size=held.size, replace=False)
    owner[pos] = held
    slot = home.copy()
    for i, f in enumerate(owner):
        if f >= 0:
            slot[f // E][f % E] = i
    scores = rng.integers(0, 6, size=(L, E)).astype(np.float32) * 0.5
    flat = scores.reshape(-1)
    ranked = sorted(range(N), key=key(scores))
    cap = int(rng.integers(1, N + 2))
    new_slot, new_owner, swaps = T.tier_rebalance(scores, n_hot, cap, home, slot, owner)
    _tier_consistent(new_slot, new_owner, home, E)
    cands = [f for f in ranked if f not in set(owner.tolist())]
    assert [sw[0] for sw in swaps] == cands[:len(swaps)] and len(swaps) <= cap
    empties_before = int((owner < 0).sum())
    assert [sw[1] for sw in swaps[:empties_before]] == [-1] * min(empties_before, len(swaps))
    residents = [int(f) for f in new_owner if f >= 0]
    left_out = [f for f in range(N) if f not in residents]
    if len(swaps) < cap and residents and len(residents) == n_hot:
        assert all(flat[f] <= min(flat[r] for r in residents) for f in left_out)
    if len(swaps) < cap and len(residents) < n_hot:
        assert not left_out  # free slots take every candidate


# ---------------------------------------------------------------- stack

def test_rms_normalize_closed_forms():
    x = np.array([[3.0, 4.0], [1e-3, -1e-3]])
    # mean square of (3, 4) is 12.5
    np.testing.assert_allclose(O.rms_normalize(x, 0.0)[0], [3 / np.sqrt(12.5), 4 / np.sqrt(12.5)], rtol=1e-15)
    rng = np.random.default_rng(0)
    z = rng.normal(size=(5, 64)) * 7.0
    n = O.rms_normalize(z, 0.0)
    np.testing.assert_allclose(np.mean(n * n, axis=1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(O.rms_normalize(3.5 * z, 0.0), n, rtol=1e-13)  # scale invariance
    # eps only matters for tiny vectors: mean square 1e-6, eps 1e-6 halves it
    np.testing.assert_allclose(O.rms_normalize(x[1:], 1e-6), x[1:] / np.sqrt(2e-6), rtol=1e-12)


def test_stack_chaining_and_identity():
    rng = np.random.default_rng(4)
    T, H, E, L, k = 2, 6, 5, 3, 2
    x = rng.normal(size=(T, H))
    Wr = rng.normal(size=(L, E, H))
    getters = [_scaled_identity_experts(rng.normal(size=E + 1), rng.normal(size=E + 1), H) for _ in range(L)]
    xo, idx, w, hist = O.moe_stack_decode(x, Wr, None, k, getters, E)
    assert np.array_equal(hist[0], x)
    for l in range(L):
        xn = hist[l] / np.sqrt(np.mean(hist[l] ** 2, axis=1, keepdims=True) + 1e-6)
        y, i2, w2, _, _ = O.moe_layer(xn, Wr[l], None, k, getters[l], E)
        nxt = hist[l + 1] if l + 1 < L else xo
        np.testing.assert_array_equal(nxt, hist[l] + y)
        assert np.array_equal(i2, idx[l])
    zero = [_scaled_identity_experts(np.ones(E + 1), np.zeros(E + 1), H)] * L
    xo, *_ = O.moe_stack_decode(x, Wr, None, k, zero, E)
    np.testing.assert_array_equal(xo, x)


def test_pages_structural_constants():
    with open(os.path.join(GOLD, "pages_constants.json")) as f:
        c = json.load(f)
    assert c["layers"] * c["experts_per_layer"] == c["total_experts"]
    assert c["layers"] * c["top_k"] == c["experts_per_token"]
    # one token's routed rows over 48 layers: permuting a single token per
    # layer gives exactly k rows per layer, all distinct experts
    idx = np.arange(c["top_k"])[None, :]
    counts, *_ = O.permute(idx, c["experts_per_layer"])
    assert counts.sum() == c["top_k"] and counts.max() == 1


# ---------------------------------------------------------------- number formats and the slot table

def test_bf16_to_f64_hand_picked_patterns():
    """bf16 is the top half of an IEEE binary32 word: each pattern is checked
    against Python's own binary32 decoder (struct) and against hand-derived
    values, including sign handling of int16 inputs."""
    cases = {
        0x3F80: 1.0, 0xC000: -2.0, 0x0000: 0.0, 0x4049: 3.140625, 0x3E80: 0.25,
        0x0080: 2.0 ** -126,                  # smallest normal
        0x0001: 2.0 ** -133,                  # smallest subnormal: 2^-126 * 2^-7
        0x007F: 127 * 2.0 ** -133,            # largest subnormal
        0x7F7F: (2 - 2 ** -7) * 2.0 ** 127,   # largest finite
        0xFF7F: -(2 - 2 ** -7) * 2.0 ** 127,
        0x7F80: math.inf, 0xFF80: -math.inf,
    }
    bits = np.array(list(cases), np.uint16)
    got = O.bf16_to_f64(bits)
    for b, v, g in zip(bits, cases.values(), got):
        assert g == v, hex(int(b))
        assert g == struct.unpack(">f", bytes([int(b) >> 8, int(b) & 0xFF, 0, 0]))[0]
    neg0 = O.bf16_to_f64(np.array([0x8000], np.uint16))[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) == -1.0
    assert np.isnan(O.bf16_to_f64(np.array([0x7FC0, 0xFFC1], np.uint16))).all()
    # the same patterns given as (negative) int16, as torch stores bf16 bits
    as_i16 = bits.view(np.int16)
    assert (as_i16 < 0).any()
    np.testing.assert_array_equal(O.bf16_to_f64(as_i16), got)
    np.testing.assert_array_equal(O.bf16_to_f64(as_i16.astype(np.int64)), got)
    # every pattern agrees with torch's own bf16 widening
    allb = np.arange(1 << 16, dtype=np.uint16)
    ref = torch.from_numpy(allb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = O.bf16_to_f64(allb)
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(mine[fin], ref[fin])
    np.testing.assert_array_equal(np.isnan(mine), np.isnan(ref))


def _constant_record(H, F, q, scale_bits):
    """An int4 record whose every weight is q * scale: every nibble q + 8 and
    every fp16 scale `scale_bits`, written straight from the format text
    (q planes take the first 3HF/2 bytes, the two scale planes the rest)."""
    R = G.record_bytes(0, H, F)
    rec = np.empty(R, np.uint8)
    n = q + 8
    rec[:3 * H * F // 2] = n | (n << 4)
    rec[3 * H * F // 2:] = np.frombuffer(struct.pack("<H", scale_bits) * ((R - 3 * H * F // 2) // 2), np.uint8)
    return rec


def test_expert_getter_follows_the_slot_table():
    """Records at known slots of a padded pool: record s holds the constant
    weight (s - 8) * 2^-3 (nibbles 0..14), so every decoded matrix names the slot it came
    from.  The slot table is a non-trivial permutation of a 3 x 5 table whose
    column E = 4 is each layer's shared expert; the record stride is larger
    than a record, and the padding holds bytes that decode to other values."""
    H, F, L, E = 128, 128, 3, 4
    R0 = G.record_bytes(0, H, F)
    stride = R0 + 512
    n_slots = L * (E + 1)
    pool = np.full(n_slots * stride, 0x77, np.uint8)  # padding: nibble 7 = q -1, scale bits 0x7777
    for s in range(n_slots):
        pool[s * stride:s * stride + R0] = _constant_record(H, F, s - 8, 0x3000)  # fp16 0x3000 = 2^-3
    rng = np.random.default_rng(11)
    S = rng.permutation(n_slots).astype(np.int32).reshape(L, E + 1)
    assert not np.array_equal(S, np.arange(n_slots).reshape(L, E + 1))
    for layer in range(L):
        get = O.expert_getter(pool, S, layer, 0, H, F, stride)
        for e in range(E + 1):
            want = (int(S[layer, e]) - 8) * 0.125
            for M in get(e):
                assert M.shape in ((F, H), (H, F))
                assert np.all(M == want), (layer, e)
    # a transposed lookup S[e][layer] would read other slots
    assert any(S[l, e] != S[e, l] for l in range(L) for e in range(L))
