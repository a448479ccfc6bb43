"""A routing trace turned into a usage profile on the device, saved, loaded
and used to fill a hot tier, against the oracle at every stage (bit-exact:
the usage scores are exactly emulated fp32 arithmetic and the tier is
integer work)."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import tier as TI
from routed_expert_ffn_moe_amd import usage_io as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_ffn_moe_amd as M
    M.load(build_if_missing=False)
    return M


def _zipf_step(rng, L, T, k, E, ranks):
    """Per layer and token k distinct experts, drawn with Zipf(1.1) popularity
    over a fixed per-layer ranking (so the profile has structure)."""
    out = np.empty((L, T, k), np.int32)
    for l in range(L):
        p = ranks[l].astype(np.float64) ** -1.1
        p /= p.sum()
        for t in range(T):
            out[l, t] = rng.choice(E, size=k, replace=False, p=p)
    return out


@pytest.mark.parametrize("L,E,T,k,steps,n_hot", [(48, 512, 1, 10, 24, 4096), (4, 64, 4, 6, 9, 40)])
def test_trace_to_profile_to_tier(moe, tmp_path, L, E, T, k, steps, n_hot):
    from routed_expert_ffn_moe_amd.profile import build_profile
    rng = np.random.default_rng(L * 100 + steps)
    ranks = np.stack([rng.permutation(E) + 1 for _ in range(L)])
    trace = str(tmp_path / "trace.bin")
    recorded = []
    with U.RoutingTrace(trace, L, T, k) as tr:
        for _ in range(steps):
            ids = _zipf_step(rng, L, T, k, E, ranks)
            recorded.append(ids)
            tr.append(torch.from_numpy(ids).cuda())  # as moe_decode_stack's topk_idx_out would be dumped
    prof = str(tmp_path / "profile.bin")
    scores = build_profile(trace, E, prof, decay=0.99)
    torch.cuda.synchronize()
    ref = np.zeros((L, E), np.float32)
    for s, ids in enumerate(recorded):
        for l in range(L):
            ref, _ = O.usage_update(ref, ids[l], l, 0.99, s, 4, 1)
    assert np.array_equal(scores.cpu().numpy(), ref)
    loaded, n = U.load_profile(prof)
    assert n == steps and loaded.tobytes() == ref.tobytes()
    # fill a hot tier from the loaded profile
    R = 256
    home = (n_hot + rng.permutation(L * (E + 1))).astype(np.int32).reshape(L, E + 1)
    pool = torch.zeros((n_hot + L * (E + 1)) * R, dtype=torch.uint8, device="cuda")
    pool[n_hot * R:] = torch.from_numpy(rng.integers(0, 256, size=L * (E + 1) * R, dtype=np.uint8)).cuda()
    home_t = torch.from_numpy(home).cuda()
    slot = torch.empty_like(home_t)
    owner = torch.empty(n_hot, dtype=torch.int32, device="cuda")
    swaps = torch.empty((n_hot, 4), dtype=torch.int32, device="cuda")
    n_sw = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_tier_fill(torch.from_numpy(loaded).cuda(), n_hot, home_t, slot, owner, pool, R, swaps, n_sw)
    torch.cuda.synchronize()
    r_slot, r_owner, r_swaps = TI.tier_fill(loaded, n_hot, home)
    assert np.array_equal(slot.cpu().numpy(), r_slot)
    assert np.array_equal(owner.cpu().numpy(), r_owner)
    assert int(n_sw.item()) == len(r_swaps)
    # the hot records are byte copies of their experts' home records
    v = pool.view(-1, R)
    s = torch.from_numpy(r_slot[:, :E].reshape(-1).astype(np.int64)).cuda()
    h = torch.from_numpy(home[:, :E].reshape(-1).astype(np.int64)).cuda()
    assert torch.equal(v[s], v[h])
