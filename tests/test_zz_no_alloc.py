"""moe_decode_stack_noalloc (the entry point for callers that cannot
allocate) against moe_decode_stack, through the C ABI: two calls in a row on
the library's per-device scratch, the second with a smaller input (fewer
tokens and layers), each bit-identical to moe_decode_stack on a fresh
workspace (same kernels, same inputs), plus the kernel-chain path and the
oracle on every gap-safe token of the first layer."""
import numpy as np
import pytest
import torch

import oracle as O
from tests import cases as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_ffn_moe_amd as M
    M.load(build_if_missing=False)
    return M


def _pair(moe, li, L, T, k):
    Wr, b, S = li.Wr[:L].contiguous(), li.bias[:L].contiguous(), li.S[:L].contiguous()
    x = li.x[:T].contiguous()
    H = x.shape[1]
    out = {}
    for name in ("noalloc", "ws"):
        idx = torch.full((L, T, k), -1, dtype=torch.int32, device="cuda")
        xo = torch.full_like(x, float("nan"))
        hist = torch.empty((L, T, H), dtype=torch.float32, device="cuda")
        if name == "noalloc":
            moe.moe_decode_stack_noalloc(x, li.F, li.E, k, Wr, b, S, li.pool, li.R, li.qfmt, x_out=xo,
                                         topk_idx_out=idx, x_hist=hist)
        else:
            moe.moe_decode_stack(x, li.F, li.E, k, Wr, b, S, li.pool, li.R, li.qfmt, x_out=xo, topk_idx_out=idx,
                                 x_hist=hist)
        torch.cuda.synchronize()
        out[name] = (xo, idx, hist)
    return x, out


@pytest.mark.parametrize("path", ["auto", "chain"])
def test_noalloc_matches_workspace_entry_point(moe, path, monkeypatch):
    if path == "chain":
        monkeypatch.setenv("MOE_DECODE_PATH", "chain")
    k = 10
    li = C.layer_case(21, 4, 2048, 512, k, 768, bias=True, L=4, device="cuda")
    for L, T in [(4, 4), (2, 1)]:
        x, out = _pair(moe, li, L, T, k)
        (xa, ia, ha), (xb, ib, hb) = out["noalloc"], out["ws"]
        assert torch.isfinite(xa).all()
        assert torch.equal(xa, xb) and torch.equal(ia, ib) and torch.equal(ha, hb), (path, L, T)
        # layer 0 against the oracle (its tokens are gap-safe by construction)
        xn = torch.from_numpy(O.rms_normalize(C.x_as_f64(x)))
        ry, ri, _, _, _ = C.oracle_layer(li, layer=0, x=xn)
        assert np.array_equal(ia[0].cpu().numpy(), ri)
        nxt = ha[1] if L > 1 else xa
        C.assert_close_moe((nxt - x).cpu().numpy(), ry, f"layer 0 (L={L}, T={T})")


def test_noalloc_rejects_oversized(moe):
    """An 8-token window of the full shape needs more scratch than the
    reserved array: rejected before anything is enqueued."""
    T, H, E, k, F = 8, 2048, 512, 8, 768
    assert moe.moe_workspace_size(moe.MOE_OP_DECODE_STACK, T, k, E, H, F, 0) > 24 << 20
    x = torch.zeros((T, H), device="cuda")
    Wr = torch.zeros((1, E, H), dtype=torch.int16, device="cuda")
    S = torch.zeros((1, E + 1), dtype=torch.int32, device="cuda")
    R = moe.moe_record_bytes(0, H, F)
    pool = torch.zeros(R, dtype=torch.uint8, device="cuda")
    xo = torch.full_like(x, 7.0)
    with pytest.raises(moe.MoeError, match="no-alloc"):
        moe.moe_decode_stack_noalloc(x, F, E, k, Wr, None, S, pool, R, 0, x_out=xo)
    torch.cuda.synchronize()
    assert bool((xo == 7.0).all())  # nothing ran
