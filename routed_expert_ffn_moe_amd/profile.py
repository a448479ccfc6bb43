"""Usage profile from a routing trace, built on the device.

The pages' engine lets a user build a personal expert ranking: run once with
the routing dump switched on, then feed the trace to a profile tool, whose
output fills the expert cache at the next start ("Strata 原理图解12GB 显卡如何
塞下 125B MoE 模型还写出 93 tokens/s", the expert-cache part; "Strata：12GB 显卡
跑 125B 模型，MoE 专家热缓存打破 VRAM 限制", section "How It Works": the usage
distribution is saved and reloaded so a restart skips the cold start).

build_profile replays a trace written by usage_io.RoutingTrace through
moe_usage_update_stack, one launch per traced step (exactly the decayed
usage update a live run performs after each step), and optionally writes the
result with usage_io.save_profile.  The profile then fills a hot tier with
moe_tier_fill.

    python -m routed_expert_ffn_moe_amd.profile TRACE PROFILE --experts 512 [--decay 0.99]
"""
import argparse

import numpy as np
import torch

from . import ops, usage_io

__all__ = ["build_profile"]


def build_profile(trace_path, E, out_path=None, decay=0.99, device="cuda", scores=None):
    """Replays the trace through moe_usage_update_stack.  Returns the scores
    fp32 [L][E] on `device` (starting from `scores`, or zeros) and, with
    out_path, saves them together with the number of steps replayed."""
    steps = usage_io.read_routing_trace(trace_path)  # int32 [n][L][T][k]
    n, L, T, k = steps.shape
    if scores is None:
        scores = torch.zeros((L, E), dtype=torch.float32, device=device)
    elif tuple(scores.shape) != (L, E):
        raise ValueError(f"scores of shape {tuple(scores.shape)}, trace has {L} layers of {E} experts")
    hits = torch.empty((L, E), dtype=torch.int32, device=device)
    ids = torch.from_numpy(steps).to(device)
    for s in range(n):
        ops.moe_usage_update_stack(ids[s], E, decay, s, 1, 1, hits, scores)  # no top_out: no re-rank
    if out_path is not None:
        usage_io.save_profile(out_path, scores, n)
    return scores


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("trace")
    ap.add_argument("profile")
    ap.add_argument("--experts", type=int, required=True, help="routed experts per layer (E)")
    ap.add_argument("--decay", type=float, default=0.99)
    a = ap.parse_args(argv)
    s = build_profile(a.trace, a.experts, a.profile, a.decay)
    top = np.argsort(-s.cpu().numpy().reshape(-1), kind="stable")[:8]
    print(f"profile of {s.shape[0]} x {s.shape[1]} experts written to {a.profile}; "
          f"top experts (layer, expert): {[(int(i) // a.experts, int(i) % a.experts) for i in top]}")


if __name__ == "__main__":
    main()
