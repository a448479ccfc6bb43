"""Per-phase timing of the persistent decode kernel.

    python -m routed_expert_ffn_moe_amd.phase_stamps build
    python -m routed_expert_ffn_moe_amd.phase_stamps run [T ...] [--qfmt 0|1]

`build` compiles the library a second time with MOE_PT_STAMPS defined (thread
0 of every workgroup then records the 100 MHz wall clock at each phase
boundary of layers < 64) into libmoe_stamps.so next to this file; the normal
library is not touched.  `run` loads that library instead of libmoe.so, runs
the 48-layer int4 (or int2) decode stack at each T on synthetic inputs (5
untimed steps, then one timed step whose stamps are read back) and prints the
per-phase times averaged over layers 1..47 and the workgroups, with the mean
over layers of the slowest workgroup's time in each phase.

Stamps per layer (index: boundary): 0 layer start, 1 x_l received, 10 1/rms,
11 router rows published, 2 x_l prepared, 3 logits received, 4 top-k done,
5 gate/up dots done, 6 SiLU done, 7 group done, 8 partial sums received,
9 layer done, 15 first group done, 12 the second group's gate/up dots done,
13 the plan done (several tokens), and 14 the workgroup's group count.  With several groups per workgroup, 5-7 are those of its last
group (the gate/up phase then spans the earlier groups).
"""
import argparse
import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
STAMP_LIB = os.path.join(HERE, "libmoe_stamps.so")
PHASES = [("wait x", 0, 1), ("router+prep", 1, 2), ("wait logits", 2, 3), ("top-k", 3, 4),
          ("gate/up", 4, 5), ("silu", 5, 6), ("down", 6, 7), ("wait partials", 7, 8), ("final", 8, 9)]
DETAIL = [("1/rms", 1, 10), ("router dot+put", 10, 11), ("xprep", 11, 2)]
NSTAMP, MAXL, MAXG = 16, 64, 256


def build():
    from . import build as B
    saved = (B.BUILD, B.LIB, B.CFLAGS)
    try:
        B.BUILD = os.path.join(HERE, "_build_stamps")
        B.LIB = STAMP_LIB
        B.CFLAGS = B.CFLAGS + ["-DMOE_PT_STAMPS"]
        return B.build()
    finally:
        B.BUILD, B.LIB, B.CFLAGS = saved


def run(ts, qfmt=0, L=48, E=512, H=2048, F=768, k=10, seed=2):
    import numpy as np
    import torch
    from . import _lib
    if not os.path.exists(STAMP_LIB):
        raise SystemExit(f"{STAMP_LIB} is missing: run `python -m routed_expert_ffn_moe_amd.phase_stamps build`")
    _lib.LIB_PATH = STAMP_LIB
    from . import ops as M
    sys.path.insert(0, os.path.dirname(HERE))
    import gen as G
    lib = _lib.load(build_if_missing=False)
    if not hasattr(lib, "moe_pt_read_stamps"):
        raise SystemExit("the loaded library was not built with MOE_PT_STAMPS")
    lib.moe_pt_read_stamps.restype = ctypes.c_int
    lib.moe_pt_read_stamps.argtypes = [ctypes.c_void_p]
    dev = torch.device("cuda:0")
    li = G.make_layer_inputs(seed, L, E, H, F, qfmt=qfmt, bias=True, device=dev)
    out = []
    for T in ts:
        ws = M.workspace(M.MOE_OP_DECODE_STACK, dev, T, k, E, H, F, qfmt)
        xo = torch.empty((T, H), device=dev)
        for rep in range(6):
            x = G.draw_x(seed, T, H, dev, tag=f"stamps{rep}")
            if rep == 5:
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
            M.moe_decode_stack(x, F, E, k, li.Wr, li.bias, li.S, li.pool, li.R, qfmt, x_out=xo, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        buf = np.zeros(MAXL * MAXG * NSTAMP, np.uint64)
        rc = lib.moe_pt_read_stamps(buf.ctypes.data_as(ctypes.c_void_p))
        st = buf.reshape(MAXL, MAXG, NSTAMP)[:L].astype(np.int64)
        ng = int((st[0, :, 0] > 0).sum())  # workgroups that stamped
        st = st[:, :ng]
        lines = [f"T={T} qfmt={qfmt}: step {e0.elapsed_time(e1) * 1e3:.0f} us (read-back rc {rc}), "
                 f"{ng} workgroups; layer {((st[1:, :, 9] - st[1:, :, 0]) / 100.0).mean():.2f} us (mean over layers 1..{L - 1} and workgroups)"]
        for name, i, j in PHASES:
            d = (st[1:, :, j] - st[1:, :, i]) / 100.0
            lines.append(f"  {name:14s} {d.mean():6.2f} us   (slowest workgroup, mean over layers {d.max(axis=1).mean():6.2f})")
        for name, i, j in DETAIL:
            d = (st[1:, :, j] - st[1:, :, i]) / 100.0
            lines.append(f"    {name:18s} {d.mean():6.2f} us")
        # the group phase (top-k done -> last group done) against the workgroup's group count
        ng_wg = st[1:, :, 14]
        gp = (st[1:, :, 7] - st[1:, :, 4]) / 100.0
        parts = []
        for n in sorted(set(ng_wg.ravel().tolist())):
            sel = ng_wg == n
            parts.append(f"{n} groups: {sel.mean() * 100:.0f}% of workgroups, {gp[sel].mean():.2f} us")
        lines.append("  group phase by group count: " + "; ".join(parts))
        first = (st[1:, :, 15] - st[1:, :, 4]) / 100.0
        later = np.where(ng_wg > 1, (st[1:, :, 7] - st[1:, :, 15]) / np.maximum(ng_wg - 1, 1) / 100.0, np.nan)
        lines.append(f"  first group {first.mean():.2f} us, each later group {np.nanmean(later) if np.isfinite(later).any() else 0:.2f} us")
        two = ng_wg >= 2
        if two.any():
            g2 = (st[1:, :, 12] - st[1:, :, 15])[two].mean() / 100.0
            lines.append(f"  second group: start -> gate/up dots done {g2:.2f} us")
        if T > 1:
            lines.append(f"  plan (after top-k) {((st[1:, :, 13] - st[1:, :, 4]) / 100.0).mean():.2f} us")
        ends = st[1:, :, 9]
        lines.append(f"  layer-end skew across workgroups: mean {((ends.max(1) - ends.min(1)) / 100.0).mean():.2f} us")
        print("\n".join(lines), flush=True)
        out.append(lines)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("what", choices=["build", "run"])
    ap.add_argument("T", type=int, nargs="*", default=[1])
    ap.add_argument("--qfmt", type=int, default=0)
    a = ap.parse_args(argv)
    if a.what == "build":
        print(build())
    else:
        run(a.T or [1], qfmt=a.qfmt)


if __name__ == "__main__":
    main()
