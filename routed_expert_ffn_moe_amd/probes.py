"""Python side of the measurement probes (include/moe_probes.h): the device's
practical HBM streaming-read rate and MFMA-only rate."""
import ctypes

import torch

from . import _lib
from ._lib import check

__all__ = ["stream_read_gbs", "mfma_tflops"]


def _time(fn, reps):
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    fn()
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(reps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / reps


def stream_read_gbs(nbytes=4 << 30, reps=10, device="cuda"):
    """GB/s of one read of nbytes (default 4 GiB, 16x the memory-side cache)."""
    lib = _lib.load()
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=device)
    sink = torch.empty(lib.moe_probe_stream_read_blocks(), dtype=torch.int32, device=device)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run():
        check(lib.moe_probe_stream_read(ctypes.c_void_p(src.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), s))
    t = _time(run, reps)
    del src
    return nbytes / t / 1e9


def mfma_tflops(iters=20000, reps=5, device="cuda"):
    """TFLOP/s of the register-only v_mfma_f32_32x32x16_f16 loop."""
    lib = _lib.load()
    sink = torch.empty(lib.moe_probe_mfma_blocks(), dtype=torch.float32, device=device)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run():
        check(lib.moe_probe_mfma(iters, ctypes.c_void_p(sink.data_ptr()), s))
    t = _time(run, reps)
    return lib.moe_probe_mfma_flops(iters) / t / 1e12


EXCHANGE_PATTERNS = {0: "x", 1: "logits", 2: "partials"}


def exchange_us(pattern, rounds=2000, device="cuda"):
    """Microseconds per round of one all-to-all hand-off of the decode kernel
    on its own (pattern 0 x, 1 logits, 2 partial sums): the slowest
    workgroup's time over the rounds, divided by the rounds."""
    lib = _lib.load()
    G = lib.moe_probe_exchange_blocks()
    ws = torch.empty(lib.moe_probe_exchange_ws_bytes(), dtype=torch.uint8, device=device)
    ticks = torch.zeros(G, dtype=torch.int64, device=device)
    err = torch.zeros(1, dtype=torch.int32, device=device)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    check(lib.moe_probe_exchange(pattern, rounds, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                 ctypes.c_void_p(ticks.data_ptr()), ctypes.c_void_p(err.data_ptr()), s))
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise RuntimeError(f"exchange probe pattern {pattern}: {int(err.item())} workgroups timed out")
    return float(ticks.max().item()) / 100.0 / rounds
