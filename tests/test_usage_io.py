"""Usage-profile files and routing traces (host-side, no GPU)."""
import os

import numpy as np
import pytest

from routed_expert_ffn_moe_amd import usage_io as U


def test_profile_round_trip_is_bit_exact(tmp_path):
    rng = np.random.default_rng(0)
    s = rng.uniform(0, 100, size=(48, 512)).astype(np.float32)
    s[3, 7] = np.float32(1e-45)   # a denormal survives
    s[5, 0] = -0.0
    p = str(tmp_path / "prof.bin")
    U.save_profile(p, s, 1234)
    got, step = U.load_profile(p)
    assert step == 1234 and got.dtype == np.float32
    assert got.tobytes() == s.tobytes()
    assert os.path.getsize(p) == 8 + 16 + 4 * 48 * 512
    assert not [f for f in os.listdir(tmp_path) if ".tmp" in f]  # the temporary file was renamed


def test_profile_rejects_foreign_or_short_files(tmp_path):
    p = str(tmp_path / "x.bin")
    open(p, "wb").write(b"NOTAPROF" + bytes(16))
    with pytest.raises(ValueError):
        U.load_profile(p)
    U.save_profile(p, np.ones((2, 3), np.float32), 0)
    data = open(p, "rb").read()
    open(p, "wb").write(data[:-4])
    with pytest.raises(ValueError):
        U.load_profile(p)


def test_routing_trace_append_and_read(tmp_path):
    rng = np.random.default_rng(1)
    p = str(tmp_path / "trace.bin")
    steps = [rng.integers(0, 512, size=(48, 2, 10)).astype(np.int32) for _ in range(5)]
    with U.RoutingTrace(p, 48, 2, 10) as tr:
        for s in steps:
            tr.append(s)
        with pytest.raises(ValueError):
            tr.append(np.zeros((48, 1, 10), np.int32))
    got = U.read_routing_trace(p)
    assert got.shape == (5, 48, 2, 10) and np.array_equal(got, np.stack(steps))
    open(p, "ab").write(b"\x01\x02\x03")  # a step cut short by a crash is dropped
    assert U.read_routing_trace(p).shape[0] == 5


def test_profile_snapshots_every_n_steps_and_on_close(tmp_path):
    p = str(tmp_path / "snap.bin")
    s = np.zeros((2, 4), np.float32)
    snap = U.ProfileSnapshots(p, s, every_steps=3)
    for i in range(7):
        s[0, 0] = i
        snap.step_done()
        if i + 1 == 3:
            assert U.load_profile(p)[1] == 3
    assert U.load_profile(p)[1] == 6 and U.load_profile(p)[0][0, 0] == 5
    snap.close()
    got, step = U.load_profile(p)
    assert step == 7 and got[0, 0] == 6
