#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE-FFN layer on one MI355X.

Headline (the JSON `value`): decode tokens/s through a 48-layer MoE-only stack
(512 experts top-10 + 1 shared expert per layer, hidden 2048, FFN 768, int4
blocks of 32 with fp16 scales, Zipf(1.1) router bias), batch 1, every weight
resident in HBM behind the (layer, expert) -> slot table.  One step = one
token through all 48 layers (router, top-k, expert gather-GEMV, combine),
the timed steps enqueued as one HIP graph.  Inputs are synthetic and seeded (gen/).

Also measured and reported under "extra": the speculative-verify step (4
tokens per step) and one 8,192-token prefill chunk through one layer (route,
permute, grouped GEMM on the matrix cores, combine).  On request:
  --sweep  verify windows of 1..8 token positions at top-10, and top-6;
  --int2   the int2 stack: decode at 1 and 4 tokens, a 16,384-token chunk;
  --tier   a hot tier of 4,096 expert slots: hit rate on a synthetic trace;
  --c2     one decode layer timed on its own, rotated over the 48 layers;
  --ceilings  the device's practical HBM read and MFMA rates and the decode
              kernel's all-to-all hand-offs on their own (probe kernels);
  --cold-cache  T=1 steps one by one, as they come and after evicting the
              caches (the per-step router and shared-expert bytes then come
              from HBM).
The int2 run also takes one 16,384-token chunk through all 48 layers, with
the usage update of every layer.  The CPU baseline times the oracle on the
decode step and on a sample of the prefill chunk's expert groups.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--sweep] [--int2] [--tier] [--c2] [--ceilings]
                    [--cold-cache]
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
MFMA_F16_PEAK_TFS = 2500.0  # MI355X dense fp16 / bf16 matrix peak

METRIC = "MoE decode tokens/s over 48 layers (HBM GB/s, % peak); prefill tok/s (% MFMA)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the sources that make up the persistent decode kernel
DECODE_SOURCES = ("decode_persistent_kernel.h", "decode_persistent.hip", "moe_common.h", "moe_kernels.h")


def source_hash(files=DECODE_SOURCES):
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(ROOT, "routed_expert_ffn_moe_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_tag, per_launch_units):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was
    taken on the current sources of that kernel; else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel_tag}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_hash") != source_hash(tuple(d.get("source_files", DECODE_SOURCES))):
        return None
    return d.get("bytes_per_" + per_launch_units)


class LazyPool:
    def __init__(self, pool):
        self.pool = pool

    def __getitem__(self, sl):
        return self.pool[sl].cpu().numpy()


def cpu_baseline(li, x_tok, budget_s):
    """The oracle (as it stands) on the host: the T tokens of x_tok [T][H]
    (one decode step, or a verify window) through as many of the 48 layers as
    fit in the time budget (at least 2), scaled to 48 layers."""
    import numpy as np
    import oracle as O
    S = li.S.cpu().numpy()
    x = x_tok.detach().cpu().double().numpy()
    t0, c0 = time.perf_counter(), os.times()
    n = 0
    while n < li.L and (n < 2 or time.perf_counter() - t0 < budget_s):
        Wr = O.bf16_to_f64(li.Wr[n].cpu().numpy())
        b = None if li.bias is None else li.bias[n].cpu().double().numpy()
        get = O.expert_getter(LazyPool(li.pool), S, n, li.qfmt, li.H, li.F, li.R)
        y, *_ = O.moe_layer(O.rms_normalize(x), Wr, b, li.k, get, li.E)
        x = x + y
        n += 1
    wall = time.perf_counter() - t0
    c1 = os.times()
    cpu = (c1.user - c0.user) + (c1.system - c0.system)
    per_step = wall / n * li.L
    T = x.shape[0]
    what = "1 token" if T == 1 else f"a window of {T} tokens"
    return {"value": round(T / per_step, 6), "unit": "tokens/s" if T == 1 else "token positions/s",
            "cores": round(cpu / wall, 2), "cores_available": os.cpu_count(), "kind": "oracle",
            "sample": f"{what} through the first {n} of {li.L} layers (fp64 NumPy, records decoded per layer), "
                      f"{wall:.1f} s, scaled to {li.L} layers"}, np


def host_info():
    """The host the oracle runs on: CPU model, logical cores, BLAS library and threads."""
    info = {"cpu_count": os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        import threadpoolctl
        info["blas"] = [{"api": d.get("internal_api"), "version": d.get("version"), "threads": d.get("num_threads")}
                        for d in threadpoolctl.threadpool_info() if d.get("user_api") == "blas"]
    except Exception as e:  # threadpoolctl missing or failing: say so
        info["blas"] = f"unknown ({type(e).__name__})"
    return info


def prefill_cpu_baseline(li, x_bf16, idx, budget_s):
    """The oracle on a sample of one prefill chunk through layer 0: the
    routed experts' whole groups (in expert order, until half the budget is
    used), the shared expert on 256 tokens and the router + top-k on 256
    tokens, each timed and extrapolated to the chunk (every routed row, the
    shared expert on every token, the router on every token)."""
    import numpy as np
    import oracle as O
    T, k = idx.shape
    E = li.E
    S = li.S.cpu().numpy()
    xf = x_bf16.detach().cpu().to(dtype=__import__("torch").float64).numpy()
    ids = idx.detach().cpu().numpy()
    c0 = os.times()
    t_all = time.perf_counter()
    get = O.expert_getter(LazyPool(li.pool), S, 0, li.qfmt, li.H, li.F, li.R)
    rows_done, t_routed, n_exp = 0, 0.0, 0
    t0 = time.perf_counter()
    for e in range(E):
        toks = np.nonzero((ids == e).any(axis=1))[0]
        if toks.size:
            O.expert_ffn(*get(e), xf[toks])
            rows_done += toks.size
            n_exp += 1
        t_routed = time.perf_counter() - t0
        if t_routed > budget_s / 2:
            break
    sample = np.arange(min(256, T))
    t0 = time.perf_counter()
    O.expert_ffn(*get(E), xf[sample])
    t_shared = (time.perf_counter() - t0) / sample.size
    Wr = O.bf16_to_f64(li.Wr[0].cpu().numpy())
    t0 = time.perf_counter()
    O.topk_select(O.router_logits(xf[sample], Wr), k)
    t_router = (time.perf_counter() - t0) / sample.size
    wall = time.perf_counter() - t_all
    c1 = os.times()
    est = t_routed / rows_done * (T * k) + (t_shared + t_router) * T
    return {"value": round(T / est, 3), "unit": "tokens/s", "kind": "oracle",
            "cores": round(((c1.user - c0.user) + (c1.system - c0.system)) / wall, 2),
            "sample": f"{n_exp} whole expert groups ({rows_done:,} of {T * k:,} routed rows), the shared expert and "
                      f"the router on {sample.size} tokens; {wall:.1f} s, extrapolated to the {T:,}-token chunk",
            "est_s_per_chunk": round(est, 1)}


def decode_bench(M, li, T, steps, warmup, use_graph, seed_tag, k=None):
    """Times `steps` decode steps of T tokens (top-k, li.k by default).
    Returns a dict of results."""
    import torch
    import gen as G
    dev = li.pool.device
    L, E, H, F = li.L, li.E, li.H, li.F
    k = li.k if k is None else k
    xs = G.draw_x(2, (steps + warmup) * T, H, dev, tag=seed_tag).view(steps + warmup, T, H)
    x_out = torch.empty((T, H), dtype=torch.float32, device=dev)
    idx_out = torch.empty((L, T, k), dtype=torch.int32, device=dev)
    ws = M.workspace(M.MOE_OP_DECODE_STACK, dev, T, k, E, H, F, li.qfmt)

    def step(x_in):  # every step reads its own input, resident in HBM
        M.moe_decode_stack(x_in, F, E, k, li.Wr, li.bias, li.S, li.pool, li.R, li.qfmt, x_out=x_out,
                           topk_idx_out=idx_out, ws=ws)

    last = xs[warmup + steps - 1]
    step(last)
    torch.cuda.synchronize()
    ref = x_out.clone()
    if not torch.isfinite(ref).all():
        raise RuntimeError("decode step produced non-finite values")
    for i in range(warmup):
        step(xs[i])
    graph = None
    if use_graph:
        # one graph holds all the timed steps: no per-step launch from the host
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                for i in range(steps):
                    step(xs[warmup + i])
        torch.cuda.current_stream().wait_stream(s)
        for rep in range(2):  # the replay's last step must match the eager step bit for bit
            x_out.zero_()
            graph.replay()
            torch.cuda.synchronize()
            if not torch.equal(x_out, ref):
                raise RuntimeError("graph replay differs from the eager step")
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    if graph is not None:
        graph.replay()
    else:
        for i in range(steps):
            step(xs[warmup + i])
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    # distinct experts per layer of every timed step (re-run untimed to read the routing)
    uniq = []
    for i in range(steps):
        step(xs[warmup + i])
        torch.cuda.synchronize()
        ids = idx_out.cpu()
        uniq.append([len(set(ids[l].reshape(-1).tolist())) for l in range(L)])
    return {"ms": ms, "uniq": uniq, "steps": steps, "T": T}


def decode_sweep(M, li, steps, warmup, use_graph):
    """Verify windows of 1..8 token positions at top-10, and T = 1, 4, 6 at
    top-6: ms per step, token positions per second, distinct experts per
    layer and the HBM rate of the algorithmic bytes."""
    rows = []
    for T, k in [(1, 10), (2, 10), (3, 10), (4, 10), (5, 10), (6, 10), (8, 10), (1, 6), (4, 6), (6, 6)]:
        d = decode_bench(M, li, T, steps, warmup, use_graph, f"sweep-x{T}-{k}", k=k)
        ms = d["ms"] / steps
        b = sum(decode_bytes(li, u, T) for u in d["uniq"]) / len(d["uniq"])
        u = sum(sum(x) for x in d["uniq"]) / (len(d["uniq"]) * li.L)
        row = {"T": T, "k": k, "ms_per_step": round(ms, 4), "token_positions_per_s": round(T / (ms / 1e3), 1),
               "mean_distinct_experts_per_layer": round(u, 2), "gbs": round(b / (ms / 1e3) / 1e9, 1),
               "path": "persistent"}
        log(f"sweep: {json.dumps(row)}")
        rows.append(row)
    return rows


TIER_HOT = 4096  # hot slots: 16.7% of the 24,576 routed experts


def tier_bench(M, li, steps, profile_steps=16, top_n=96, every=4, decay=0.99):
    """Capacity-limited hot tier on a synthetic trace: the tier is filled from
    a usage profile of `profile_steps` decode steps on plain N(0,1) tokens,
    then `steps` decode steps run on tokens shifted by a fixed seeded "topic"
    vector (x = z + v), with the usage update of all layers after each step
    (moe_usage_update_stack) and a rebalance
    of at most top_n swaps (the best non-resident experts) every `every`
    steps.  Hit rate = the share of the
    routed (layer, token, choice) lookups whose slot is a hot slot."""
    import torch
    import gen as G
    dev = li.pool.device
    L, E, H, F, k, R = li.L, li.E, li.H, li.F, li.k, li.R
    n_hot = TIER_HOT
    home = li.S.to(torch.int32).contiguous()
    slot = home.clone()
    owner = torch.full((n_hot,), -1, dtype=torch.int32, device=dev)
    swaps = torch.empty((max(n_hot, 1024), 4), dtype=torch.int32, device=dev)
    n_sw = torch.zeros(1, dtype=torch.int32, device=dev)
    scores = torch.zeros((L, E), dtype=torch.float32, device=dev)
    hits_ws = torch.empty((L, E), dtype=torch.int32, device=dev)
    x_in = torch.empty((1, H), dtype=torch.float32, device=dev)
    idx = torch.empty((L, 1, k), dtype=torch.int32, device=dev)
    ws = M.workspace(M.MOE_OP_DECODE_STACK, dev, 1, k, E, H, F, li.qfmt)

    def step(x, st):
        x_in.copy_(x)
        M.moe_decode_stack(x_in, F, E, k, li.Wr, li.bias, slot, li.pool, R, li.qfmt, topk_idx_out=idx, ws=ws)
        hot = (torch.gather(slot[:, :E], 1, idx.view(L, k).long()) < n_hot).sum()
        M.moe_usage_update_stack(idx, E, decay, st, every, top_n, hits_ws, scores)
        return hot

    xs = G.draw_x(7, profile_steps, H, dev, tag="tier-profile")
    for i in range(profile_steps):
        step(xs[i:i + 1], i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    M.moe_tier_fill(scores, n_hot, home, slot, owner, li.pool, R, swaps, n_sw)
    e1.record()
    torch.cuda.synchronize()
    fill_ms = e0.elapsed_time(e1)
    v = G.draw_x(7, 1, H, dev, tag="tier-topic")
    xs = G.draw_x(7, steps, H, dev, tag="tier-run") + v
    hot_per_step, swaps_per, reb_ms = [], [], []
    for i in range(steps):
        reb = (i + 1) % every == 0
        hot_per_step.append(step(xs[i:i + 1], i))
        if reb:
            e0.record()
            M.moe_tier_rebalance(scores, n_hot, top_n, home, slot, owner, li.pool, R, swaps, n_sw)
            e1.record()
            torch.cuda.synchronize()
            reb_ms.append(e0.elapsed_time(e1))
            swaps_per.append(int(n_sw.item()))
    hr = [float(h.item()) / (L * k) for h in hot_per_step]
    q = max(1, steps // 4)
    return {"hot_slots": n_hot, "hot_share_of_experts": round(n_hot / (L * E), 4),
            "profile_steps": profile_steps, "trace": "decode T=1, x = N(0,1) + a fixed N(0,1) topic vector",
            "hit_rate_first_4_steps": round(sum(hr[:4]) / 4, 4),
            "hit_rate_last_quarter": round(sum(hr[-q:]) / q, 4),
            "swaps_per_rebalance_mean": round(sum(swaps_per) / max(1, len(swaps_per)), 1),
            "rebalance_ms_mean": round(sum(reb_ms) / max(1, len(reb_ms)), 4),
            "fill_ms": round(fill_ms, 2), "fill_gb_copied": round(n_hot * R / 1e9, 2)}


def int2_bench(M, steps, warmup, use_graph, cpu_budget=None):
    """The int2 stack (blocks of 16 with fp16 scale and min; seed 4, Zipf
    routing bias): decode at T = 1 and 4 through 48 layers, and one 16,384-token
    prefill chunk through layer 0 with the bias (skewed groups); with a
    cpu_budget, the oracle on a sample of that chunk's layer (per layer, and
    scaled to the 48 layers)."""
    import torch
    import gen as G
    L, E, H, F, k = 48, 512, 2048, 768, 10
    li = G.make_layer_inputs(4, L, E, H, F, qfmt=1, bias=True, device=torch.device("cuda:0"))
    li.k = k
    out = {"pool_gb": round(li.pool.numel() / 1e9, 2), "record_bytes": li.R}
    for T in (1, 4):
        d = decode_bench(M, li, T, steps, warmup, use_graph, f"int2-x{T}")
        ms = d["ms"] / steps
        b = sum(decode_bytes(li, u, T) for u in d["uniq"]) / len(d["uniq"])
        out[f"decode_t{T}"] = {"ms_per_step": round(ms, 4), "token_positions_per_s": round(T / (ms / 1e3), 1),
                               "gbs": round(b / (ms / 1e3) / 1e9, 1),
                               "hbm_frac": round(b / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
    out["prefill_16k"] = prefill_bench(M, li, reps=5, warmup=2, T=16384, seed=4, use_bias=True)
    out["prefill_16k_48_layers"] = prefill_stack_bench(M, li, T=16384, seed=4, reps=1)
    if cpu_budget:
        xp = G.draw_x(4, 16384, H, li.pool.device, tag="bench-prefill").to(torch.bfloat16)
        idx_p, _ = M.moe_route_topk(xp, li.Wr[0].contiguous(), li.bias[0].contiguous(), k)
        pc = prefill_cpu_baseline(li, xp, idx_p, cpu_budget)
        pc["est_s_per_48_layer_chunk"] = round(pc["est_s_per_chunk"] * L, 1)
        pc["sample"] += f"; x {L} layers: {pc['est_s_per_48_layer_chunk']} s per chunk (extrapolated)"
        out["prefill_16k"]["cpu_baseline"] = pc
    del li
    torch.cuda.empty_cache()
    return out


def decode_bytes(li, uniq_step, T):
    """Algorithmic HBM bytes of one step: every distinct expert's record plus
    the shared expert's, the router matrix, and the activations read and
    written (x in, x out) per layer."""
    return sum((u + 1) * li.R + li.E * li.H * 2 + 2 * T * li.H * 4 for u in uniq_step)


def prefill_bench(M, li, reps, warmup, T=8192, seed=3, use_bias=False):
    """One T-token bf16 chunk through layer 0 (without the routing bias:
    near-uniform routing; with it: Zipf-skewed groups, some empty)."""
    import torch
    import gen as G
    dev = li.pool.device
    H, E, k, F = li.H, li.E, li.k, li.F
    x = G.draw_x(seed, T, H, dev, tag="bench-prefill").to(torch.bfloat16)
    Wr0 = li.Wr[0].contiguous()
    b0 = li.bias[0].contiguous() if use_bias else None
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    ws_r = M.workspace(M.MOE_OP_ROUTE_TOPK, dev, T=T, E=E)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_src = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv_row = torch.empty(T * k, dtype=torch.int32, device=dev)
    ws_p = M.workspace(M.MOE_OP_PERMUTE, dev, T=T, k=k, E=E)
    y_perm = torch.empty((T * k, H), dtype=torch.float16, device=dev)  # the expert rows as fp16
    y_sh = torch.empty((T, H), dtype=torch.float16, device=dev)
    ws_g = M.workspace(M.MOE_OP_GROUPED_GEMM_Q, dev, T, k, E, H, F, li.qfmt)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream()
    names = ["route", "permute", "grouped_gemm", "combine"]
    ops = [
        lambda: M.moe_route_topk(x, Wr0, b0, k, topk_idx=idx, topk_w=w, ws=ws_r),
        lambda: M.moe_permute(idx, E, counts, offsets, row_src, inv_row, ws=ws_p),
        lambda: M.moe_grouped_gemm_q(x, row_src, offsets, k, E, F, li.S, 0, li.pool, li.R, li.qfmt, y_perm=y_perm,
                                     y_shared=y_sh, ws=ws_g),
        lambda: M.moe_combine(y_perm, w, inv_row=inv_row, y_shared=y_sh, y_out=y),
    ]
    for _ in range(warmup):
        for op in ops:
            op()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(reps)]
    for r in range(reps):
        ev[r][0].record(st)
        for i, op in enumerate(ops):
            op()
            ev[r][i + 1].record(st)
    torch.cuda.synchronize()
    per_op = {n: sorted(ev[r][i].elapsed_time(ev[r][i + 1]) for r in range(reps))[reps // 2]
              for i, n in enumerate(names)}
    total = sorted(ev[r][0].elapsed_time(ev[r][-1]) for r in range(reps))[reps // 2]
    experts_hit = int((counts > 0).sum().item())
    flop_routed = 2.0 * T * k * 3 * H * F
    flop_shared = 2.0 * T * 3 * H * F
    gemm_s = per_op["grouped_gemm"] / 1e3
    tf_routed_equiv = (flop_routed + flop_shared) / gemm_s / 1e12
    return {
        "workload": f"{T:,}-token bf16 chunk, 1 layer, 512 experts top-10 + shared, "
                    f"{'int4' if li.qfmt == 0 else 'int2'}{', Zipf routing bias' if use_bias else ''} (median of {reps})",
        "tokens_per_s": round(T / (total / 1e3), 1),
        "ms_layer": round(total, 4),
        "ms_per_op": {n: round(v, 4) for n, v in per_op.items()},
        "grouped_gemm_tflops": round(tf_routed_equiv, 2),
        "grouped_gemm_mfma_frac": round(tf_routed_equiv / MFMA_F16_PEAK_TFS, 4),
        "grouped_gemm_gflop": {"routed": round(flop_routed / 1e9, 1), "shared": round(flop_shared / 1e9, 1)},
        "routed_gemm_target_ms": round(flop_routed / 1e9 / (0.5 * MFMA_F16_PEAK_TFS), 4),
        "experts_hit": experts_hit,
    }


def prefill_stack_bench(M, li, T, seed=4, reps=1):
    """One T-token chunk through all li.L layers as a pre-norm residual chain:
    per layer the norm (to bf16), route (with the routing bias), permute,
    grouped GEMM, combine into the residual stream and the layer's usage
    update (decay 0.99, top-96 re-rank after every 4th step).  The whole pass
    is timed (median of reps after one untimed pass)."""
    import torch
    import gen as G
    dev = li.pool.device
    L, H, E, k, F = li.L, li.H, li.E, li.k, li.F
    x0 = G.draw_x(seed, T, H, dev, tag="bench-prefill-stack")
    x = torch.empty_like(x0)
    xb = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    ws_r = M.workspace(M.MOE_OP_ROUTE_TOPK, dev, T=T, E=E)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_src = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv_row = torch.empty(T * k, dtype=torch.int32, device=dev)
    ws_p = M.workspace(M.MOE_OP_PERMUTE, dev, T=T, k=k, E=E)
    y_perm = torch.empty((T * k, H), dtype=torch.float16, device=dev)  # the expert rows as fp16
    y_sh = torch.empty((T, H), dtype=torch.float16, device=dev)
    ws_g = M.workspace(M.MOE_OP_GROUPED_GEMM_Q, dev, T, k, E, H, F, li.qfmt)
    scores = torch.zeros((L, E), dtype=torch.float32, device=dev)
    hits = torch.empty(E, dtype=torch.int32, device=dev)
    top = torch.empty(96, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream()

    def one_pass(step, ev=None):
        x.copy_(x0)
        if ev is not None:
            ev[0].record(st)
        for l in range(L):
            M.moe_rmsnorm(x, out=xb)
            M.moe_route_topk(xb, li.Wr[l], li.bias[l] if li.bias is not None else None, k, topk_idx=idx,
                             topk_w=w, ws=ws_r)
            M.moe_permute(idx, E, counts, offsets, row_src, inv_row, ws=ws_p)
            M.moe_grouped_gemm_q(xb, row_src, offsets, k, E, F, li.S, l, li.pool, li.R, li.qfmt, y_perm=y_perm,
                                 y_shared=y_sh, ws=ws_g)
            M.moe_combine(y_perm, w, inv_row=inv_row, y_shared=y_sh, residual=x, y_out=x)
            M.moe_usage_update(idx, l, L, E, 0.99, step, 4, 96, hits, scores, top)
        if ev is not None:
            ev[1].record(st)

    one_pass(0)
    torch.cuda.synchronize()
    if not torch.isfinite(x).all():
        raise RuntimeError("prefill stack produced non-finite values")
    times = []
    for r in range(reps):
        ev = [torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
        one_pass(r + 1, ev)
        torch.cuda.synchronize()
        times.append(ev[0].elapsed_time(ev[1]))
    ms = sorted(times)[len(times) // 2]
    flop = 2.0 * T * (k + 1) * 3 * H * F * L
    return {"workload": f"{T:,}-token chunk through {L} layers ({'int4' if li.qfmt == 0 else 'int2'}, routing bias), "
                        f"norm + route + permute + grouped GEMM + combine + usage update per layer",
            "ms_chunk": round(ms, 3), "ms_per_layer": round(ms / L, 4), "tokens_per_s": round(T / (ms / 1e3), 1),
            "expert_tflops_whole_pass": round(flop / (ms / 1e3) / 1e12, 1)}


def single_layer_bench(M, li, reps=8):
    """One decode layer on its own (T = 1): a one-layer persistent step on
    layer l, rotated over all li.L layers so that consecutive calls read
    different records (48 x 28.5 MB, well over the 256 MB memory-side cache);
    the timed calls are one HIP graph."""
    import torch
    import gen as G
    dev = li.pool.device
    L, E, H, F, k = li.L, li.E, li.H, li.F, li.k
    x = G.draw_x(1, 1, H, dev, tag="bench-c2")
    xo = torch.empty_like(x)
    ws = M.workspace(M.MOE_OP_DECODE_STACK, dev, 1, k, E, H, F, li.qfmt)
    layers = [(li.Wr[l:l + 1], li.bias[l:l + 1], li.S[l:l + 1]) for l in range(L)]
    idx = torch.empty((1, 1, k), dtype=torch.int32, device=dev)

    def call(l):
        Wr, b, S = layers[l]
        M.moe_decode_stack(x, F, E, k, Wr, b, S, li.pool, li.R, li.qfmt, x_out=xo, topk_idx_out=idx, ws=ws)

    for l in range(L):
        call(l)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for r in range(reps):
                for l in range(L):
                    call(l)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * L)
    b = 11 * li.R + E * H * 2 + 2 * H * 4
    return {"workload": "one decode layer (1 token, top-10 + shared, int4), a one-layer persistent step per call, "
                        f"rotated over {L} layers", "us_per_layer": round(us, 2), "bytes_per_layer": b,
            "gbs": round(b / (us / 1e6) / 1e9, 1), "hbm_frac": round(b / (us / 1e6) / 1e9 / HBM_PEAK_GBS, 4)}


def cold_cache_bench(M, li, steps=16, flush_mib=1024):
    """T = 1 decode steps timed one by one (events around each step), first
    as they come, then each after a streaming read of flush_mib MiB that
    evicts the L2s and the 256 MB memory-side cache: the router matrices
    and the shared experts (about 230 MB re-read by every step) then come
    from HBM.  The difference is what those caches save a step."""
    import torch
    import gen as G
    dev = li.pool.device
    L, E, H, F, k = li.L, li.E, li.H, li.F, li.k
    xs = G.draw_x(2, 2 * steps + 2, H, dev, tag="bench-cold").view(2 * steps + 2, 1, H)
    x_out = torch.empty((1, H), dtype=torch.float32, device=dev)
    ws = M.workspace(M.MOE_OP_DECODE_STACK, dev, 1, k, E, H, F, li.qfmt)
    flush = torch.ones(flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)

    def step(x_in):
        M.moe_decode_stack(x_in, F, E, k, li.Wr, li.bias, li.S, li.pool, li.R, li.qfmt, x_out=x_out, ws=ws)

    step(xs[0])
    step(xs[1])
    torch.cuda.synchronize()
    res = {}
    for name, cold in (("warm", False), ("cold", True)):
        times = []
        for i in range(steps):
            if cold:
                flush.sum()  # reads the whole buffer before the step
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step(xs[2 + (steps if cold else 0) + i])
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        res[name + "_ms_median"] = round(times[len(times) // 2], 4)
    del flush
    res["flush_mib"] = flush_mib
    res["cold_minus_warm_us"] = round((res["cold_ms_median"] - res["warm_ms_median"]) * 1e3, 1)
    res["workload"] = ("48-layer T=1 decode step, eager, one step per event pair (includes the two small "
                       "workspace kernels); cold: after a streaming read of flush_mib MiB")
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-graph", action="store_true", help="launch the step eagerly instead of a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the verify and prefill measurements")
    ap.add_argument("--sweep", action="store_true",
                    help="also time verify windows T = 1..8 at top-10 and T = 1, 4, 6 at top-6")
    ap.add_argument("--tier", action="store_true",
                    help="also emulate a hot tier of 4,096 expert slots (hit rate on a synthetic trace)")
    ap.add_argument("--int2", action="store_true",
                    help="also time the int2 stack: decode T = 1, 4 and a 16,384-token prefill chunk")
    ap.add_argument("--c2", action="store_true", help="also time one decode layer on its own, rotated over the layers")
    ap.add_argument("--cold-cache", action="store_true",
                    help="also time T=1 steps one by one with and without evicting the caches before each step")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the 8,192-token prefill chunk on a one-layer pool (for profiling the grouped GEMM); "
                         "prints that measurement, not the headline line")
    ap.add_argument("--ceilings", action="store_true",
                    help="also measure the practical HBM streaming-read and MFMA-only rates (probe kernels)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--copy-ref-mb", type=int, default=0,
                    help="run one plain device copy of this many MiB first (the reference kernel that scales "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE readings to bytes)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the layer scales data-parallel with a replicated expert pool (each "
              "GPU runs these kernels unchanged) and there is no multi-GPU path. Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gen as G
    import routed_expert_ffn_moe_amd as M
    M.load(build_if_missing=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_ref_mb > 0:
        n = args.copy_ref_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy reference: {args.copy_ref_mb} MiB read, {args.copy_ref_mb} MiB written")
        del src, dst

    L, E, H, F, k = 48, 512, 2048, 768, 10
    if args.prefill_only:
        li = G.make_layer_inputs(2, 1, E, H, F, qfmt=0, bias=True, device=dev)
        li.k = k
        pf = prefill_bench(M, li, reps=args.steps, warmup=args.warmup)
        print(json.dumps({"prefill_c4": pf}), flush=True)
        return
    t0 = time.perf_counter()
    li = G.make_layer_inputs(2, L, E, H, F, qfmt=0, bias=True, device=dev,
                             progress=lambda l: log(f"pool: layer {l + 1}/{L}") if (l + 1) % 8 == 0 else None,
                             hot_slots=TIER_HOT if args.tier else 0)
    li.k = k
    torch.cuda.synchronize()
    log(f"pool of {li.pool.numel() / 1e9:.1f} GB built in {time.perf_counter() - t0:.1f} s")

    d1 = decode_bench(M, li, 1, args.steps, args.warmup, not args.no_graph, "bench-x")
    ms_step = d1["ms"] / args.steps
    bytes_steps = [decode_bytes(li, u, 1) for u in d1["uniq"]]
    bytes_per_step = sum(bytes_steps) / len(bytes_steps)
    gbs = bytes_per_step / (ms_step / 1e3) / 1e9
    value = args.steps / (d1["ms"] / 1e3)
    log(f"decode T=1: {ms_step:.4f} ms/step, {value:.1f} tok/s, {gbs:.1f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of peak)")

    traffic = measured_traffic("decode_stack_t1", "step")
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int4-weights x fp16 dot2 -> fp32", "data": "synthetic",
        "config": {"workload": "48-layer MoE-only stack decode, batch 1 (1 token per step)", "layers": L,
                   "experts": E, "top_k": k, "shared_experts": 1, "hidden": H, "ffn": F,
                   "weights": "int4 blocks of 32, fp16 scale", "router_bias": "Zipf(1.1)",
                   "pool_gb": round(li.pool.numel() / 1e9, 2),
                   "launch": "one hip graph of the timed steps, each reading its own resident input"
                   if not args.no_graph else "eager, one launch per step"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "decode_persistent_kernel: one launch = one 48-layer step (router, top-k, experts, sum)",
                     "algorithmic_bytes_per_step": round(bytes_per_step)},
    }
    if not args.no_extra:
        d4 = decode_bench(M, li, 4, args.steps, args.warmup, not args.no_graph, "bench-x4")
        ms4 = d4["ms"] / args.steps
        b4 = sum(decode_bytes(li, u, 4) for u in d4["uniq"]) / len(d4["uniq"])
        u4 = sum(sum(u) for u in d4["uniq"]) / (len(d4["uniq"]) * L)
        pf = prefill_bench(M, li, reps=10, warmup=3)
        out["extra"] = {
            "verify_t4": {"token_positions_per_s": round(4 * args.steps / (d4["ms"] / 1e3), 1),
                          "ms_per_step": round(ms4, 5), "gbs": round(b4 / (ms4 / 1e3) / 1e9, 1),
                          "hbm_frac": round(b4 / (ms4 / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                          "mean_distinct_experts_per_layer": round(u4, 2)},
            "prefill_c4": pf,
        }
        log(f"verify T=4: {ms4:.4f} ms/step; prefill: {json.dumps(pf)}")
    if args.sweep:
        out.setdefault("extra", {})["decode_sweep"] = decode_sweep(M, li, min(args.steps, 32), args.warmup,
                                                                   not args.no_graph)
    if args.int2:
        i2 = int2_bench(M, args.steps, args.warmup, not args.no_graph,
                        cpu_budget=None if args.no_cpu_baseline else args.cpu_budget)
        log(f"int2: {json.dumps(i2)}")
        out.setdefault("extra", {})["int2_stack"] = i2
    if args.c2:
        c2 = single_layer_bench(M, li)
        log(f"c2: {json.dumps(c2)}")
        out.setdefault("extra", {})["single_layer_c2"] = c2
    if args.cold_cache:
        cc = cold_cache_bench(M, li)
        log(f"cold cache: {json.dumps(cc)}")
        out.setdefault("extra", {})["cold_cache"] = cc
    if args.ceilings:
        from routed_expert_ffn_moe_amd import probes
        ce = {"hbm_stream_read_gbs": round(probes.stream_read_gbs(device=dev), 1),
              "mfma_f16_register_loop_tflops": round(probes.mfma_tflops(device=dev), 1)}
        a16 = torch.randn((8192, 8192), device=dev, dtype=torch.float16)
        b16 = torch.randn((8192, 8192), device=dev, dtype=torch.float16)
        torch.matmul(a16, b16)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            torch.matmul(a16, b16)
        e1.record()
        torch.cuda.synchronize()
        ce["library_fp16_gemm_8192_tflops"] = round(2 * 8192 ** 3 * 5 / (e0.elapsed_time(e1) / 1e3) / 1e12, 1)
        # the decode kernel's three hand-offs on their own: the exchange floor of a layer
        ce["exchange_us_per_round"] = {name: round(probes.exchange_us(pat, device=dev), 3)
                                       for pat, name in probes.EXCHANGE_PATTERNS.items()}
        del a16, b16
        log(f"ceilings: {json.dumps(ce)}")
        out.setdefault("extra", {})["ceilings"] = ce
    if args.tier:
        tb = tier_bench(M, li, min(args.steps, 64))
        log(f"tier: {json.dumps(tb)}")
        out.setdefault("extra", {})["hot_tier"] = tb
    if not args.no_cpu_baseline:
        xs = G.draw_x(2, 1, H, dev, tag="bench-x")
        cb, _ = cpu_baseline(li, xs, args.cpu_budget)
        cb["host"] = host_info()
        out["cpu_baseline"] = cb
        log(f"cpu baseline: {cb}")
        if "extra" in out and "verify_t4" in out["extra"]:
            x4 = G.draw_x(2, 4, H, dev, tag="bench-x4")
            c4, _ = cpu_baseline(li, x4, args.cpu_budget / 3)
            out["extra"]["verify_t4"]["cpu_baseline"] = c4
            log(f"verify cpu baseline: {c4}")
        if "extra" in out and "prefill_c4" in out["extra"]:
            xp = G.draw_x(3, 8192, H, dev, tag="bench-prefill").to(torch.bfloat16)
            idx_p, _ = M.moe_route_topk(xp, li.Wr[0].contiguous(), None, k)
            pc = prefill_cpu_baseline(li, xp, idx_p, args.cpu_budget)
            out["extra"]["prefill_c4"]["cpu_baseline"] = pc
            log(f"prefill cpu baseline: {pc}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
