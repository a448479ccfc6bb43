"""Usage-profile persistence and routing-trace dumps (host-side file I/O).

The engine on the pages ships a usage profile that ranks every expert and
fills the card's expert slots from it ("为什么 Strata 在小显存显卡上这么快",
section "一台电脑就是一组水管"); it saves the current expert-usage
distribution every ten minutes and at exit and loads it at the next start,
skipping the cold start ("Strata：12GB 显卡跑 125B 模型，MoE 专家热缓存打破
VRAM 限制", sections "MoE 的推理特性" and "How It Works"); a user builds a
personal ranking by running once with a routing dump and feeding the trace to
a profile tool ("Strata 原理图解12GB 显卡如何塞下 125B MoE 模型还写出 93
tokens/s").  Here:

  * a profile file holds the decayed usage scores fp32 [L][E] of
    moe_usage_update and the step they were taken at;
  * a routing trace holds the chosen experts int32 [L][T][k] of every step
    (moe_decode_stack's topk_idx_out), appended step by step;
  * ProfileSnapshots saves a profile every `every_steps` steps and on close.

Formats (little-endian):
  profile: b"MOEPROF1", int32 L, int32 E, int64 step, fp32 scores[L*E]
  trace:   b"MOETRAC1", int32 L, int32 T, int32 k, int32 0, then per step
           int32 ids[L*T*k]
A profile is written to a temporary file in the same directory and renamed
over the old one, so a reader never sees a partial profile.
"""
import os
import struct

import numpy as np

__all__ = ["save_profile", "load_profile", "RoutingTrace", "read_routing_trace", "ProfileSnapshots"]

_PROFILE_MAGIC = b"MOEPROF1"
_TRACE_MAGIC = b"MOETRAC1"


def _host_array(t, dtype):
    """A torch tensor (any device) or array-like as a contiguous numpy array."""
    if hasattr(t, "detach"):
        t = t.detach().to("cpu").numpy()
    return np.ascontiguousarray(np.asarray(t, dtype=dtype))


def save_profile(path, scores, step):
    """Writes scores [L][E] (fp32) and the step they belong to."""
    s = _host_array(scores, "<f4")
    if s.ndim != 2:
        raise ValueError("scores must be [L][E]")
    L, E = s.shape
    tmp = f"{path}.tmp{os.getpid()}"
    with open(tmp, "wb") as f:
        f.write(_PROFILE_MAGIC + struct.pack("<iiq", L, E, int(step)))
        f.write(s.tobytes())
        f.flush()
        os.fsync(f.fileno())
    os.replace(tmp, path)


def load_profile(path):
    """Returns (scores numpy fp32 [L][E], step)."""
    with open(path, "rb") as f:
        head = f.read(8 + 16)
        if len(head) != 24 or head[:8] != _PROFILE_MAGIC:
            raise ValueError(f"{path}: not a usage profile")
        L, E, step = struct.unpack("<iiq", head[8:])
        if L < 1 or E < 1:
            raise ValueError(f"{path}: bad shape {L}x{E}")
        body = f.read()
    if len(body) != 4 * L * E:
        raise ValueError(f"{path}: {len(body)} bytes of scores, expected {4 * L * E}")
    return np.frombuffer(body, dtype="<f4").reshape(L, E).copy(), step


class RoutingTrace:
    """Appends the chosen experts [L][T][k] of each step to a file."""

    def __init__(self, path, L, T, k):
        self.path, self.shape = path, (L, T, k)
        self._f = open(path, "wb")
        self._f.write(_TRACE_MAGIC + struct.pack("<iiii", L, T, k, 0))

    def append(self, topk_idx):
        a = _host_array(topk_idx, "<i4")
        if a.shape != self.shape:
            raise ValueError(f"routing of shape {a.shape}, trace holds {self.shape}")
        self._f.write(a.tobytes())

    def close(self):
        if self._f is not None:
            self._f.close()
            self._f = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def read_routing_trace(path):
    """Returns int32 [steps][L][T][k]; a step cut short at the end is dropped."""
    with open(path, "rb") as f:
        head = f.read(24)
        if len(head) != 24 or head[:8] != _TRACE_MAGIC:
            raise ValueError(f"{path}: not a routing trace")
        L, T, k, _ = struct.unpack("<iiii", head[8:])
        body = f.read()
    per = 4 * L * T * k
    n = len(body) // per
    return np.frombuffer(body[:n * per], dtype="<i4").reshape(n, L, T, k).copy()


class ProfileSnapshots:
    """Saves the usage scores every `every_steps` steps and on close."""

    def __init__(self, path, scores, every_steps):
        if every_steps < 1:
            raise ValueError("every_steps must be >= 1")
        self.path, self.scores, self.every = path, scores, every_steps
        self.step = 0

    def step_done(self):
        self.step += 1
        if self.step % self.every == 0:
            save_profile(self.path, self.scores, self.step)

    def close(self):
        save_profile(self.path, self.scores, self.step)
