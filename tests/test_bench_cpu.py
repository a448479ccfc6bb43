"""bench.py's host-side arithmetic and contract (no GPU)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


class _Stack:
    L, E, H, F, k = 48, 512, 2048, 768, 10
    R = 2_654_208  # int4 record: 27 H F / 16 bytes


def test_algorithmic_bytes_of_a_one_token_step():
    """48 layers x (10 routed + 1 shared record + the 2 MiB bf16 router) plus
    x read and written per layer: the roofline's denominator."""
    per_layer = 11 * 2_654_208 + 512 * 2048 * 2 + 2 * 1 * 2048 * 4
    assert bench.decode_bytes(_Stack, [10] * 48, 1) == 48 * per_layer == 1_502_871_552


def test_algorithmic_bytes_count_distinct_experts():
    # four tokens sharing experts: only the distinct ones (plus the shared one) are read
    b = bench.decode_bytes(_Stack, [25] * 48, 4)
    assert b == 48 * (26 * 2_654_208 + 512 * 2048 * 2 + 2 * 4 * 2048 * 4)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_reported_only_for_the_profiled_sources():
    p = os.path.join(ROOT, "profiles", "decode_stack_t1_traffic.json")
    d = json.load(open(p))
    files = tuple(d["source_files"])
    assert set(files) >= {"decode_persistent_kernel.h", "decode_persistent.hip"}
    if d["source_hash"] == bench.source_hash(files):
        assert bench.measured_traffic("decode_stack_t1", "step") == d["bytes_per_step"]
        assert d["bytes_per_step"] == d["read_bytes_per_step"] + d["write_bytes_per_step"]
    else:
        assert bench.measured_traffic("decode_stack_t1", "step") is None
    assert bench.measured_traffic("no_such_kernel", "step") is None
