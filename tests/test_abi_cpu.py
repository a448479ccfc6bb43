"""CPU-side checks of the C ABI: the library loads, exports every declared
entry point, answers size queries, and rejects bad arguments with the
documented codes before launching anything (no GPU is touched).  Every call
below carries at least one invalid argument, so validation fails before any
HIP call; the dummy addresses are never dereferenced."""
import ctypes
import os
import re

import pytest

from routed_expert_ffn_moe_amd import _lib
import gen as G

HEADER = os.path.join(os.path.dirname(__file__), "..", "include", "moe.h")
PROBES = os.path.join(os.path.dirname(__file__), "..", "include", "moe_probes.h")
FAKE = 0x10000  # non-null, 256-byte aligned dummy "device" address (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions(header=HEADER):
    txt = open(header).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(moe_\w+)\s*\(", txt, flags=re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 19, names
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def test_version_and_sizes(lib):
    assert lib.moe_abi_version() == 1
    assert lib.moe_record_bytes(0, 2048, 768) == G.record_bytes(0, 2048, 768) == 2_654_208
    assert lib.moe_record_bytes(1, 2048, 768) == G.record_bytes(1, 2048, 768) == 2_359_296
    assert lib.moe_record_bytes(0, 256, 128) == 55_296
    assert lib.moe_record_bytes(0, 200, 128) == 0 and lib.moe_record_bytes(7, 256, 128) == 0
    assert lib.moe_workspace_size(_lib.MOE_OP_COMBINE, 4, 2, 16, 256, 128, 0) == 0
    assert lib.moe_workspace_size(_lib.MOE_OP_ROUTE_TOPK, 8192, 10, 512, 2048, 0, 0) >= 8192 * 512 * 4
    assert lib.moe_workspace_size(_lib.MOE_OP_GROUPED_GEMM_Q, 8192, 10, 512, 2048, 768, 0) >= 90112 * 768 * 2
    assert lib.moe_workspace_size(_lib.MOE_OP_EXPERT_GEMV_Q, 1, 10, 512, 2048, 768, 0) > 0
    assert lib.moe_workspace_size(99, 1, 1, 1, 1, 1, 0) == 0


def _err(lib):
    return lib.moe_last_error().decode()


def test_route_topk_rejects(lib):
    f = lib.moe_route_topk
    ok = dict(x=FAKE, xd=0, T=4, H=256, wr=FAKE, b=None, E=16, k=2, idx=FAKE, w=FAKE, lg=FAKE, ws=None, wsb=0, s=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["xd"], a["T"], a["H"], a["wr"], a["b"], a["E"], a["k"], a["idx"], a["w"], a["lg"],
                 a["ws"], a["wsb"], a["s"])
    assert call(k=17) == _lib.MOE_ESHAPE and "k=17" in _err(lib)
    assert call(k=20, E=16) == _lib.MOE_ESHAPE
    assert call(E=2000) == _lib.MOE_ESHAPE
    assert call(H=200) == _lib.MOE_ESHAPE
    assert call(xd=5) == _lib.MOE_EUNSUPPORTED
    assert call(x=None) == _lib.MOE_EINVAL
    assert call(x=FAKE + 4) == _lib.MOE_EALIGN
    assert call(lg=None) == _lib.MOE_EWORKSPACE           # no logits_out and no ws
    assert call(lg=None, ws=FAKE, wsb=16) == _lib.MOE_EWORKSPACE
    assert call(T=0, x=None, wr=None) == _lib.MOE_OK       # nothing to do, nothing launched


def test_expert_ops_reject(lib):
    g = lib.moe_expert_gemv_q
    base = [FAKE, 1, 2048, 768, FAKE, 10, 512, FAKE, 0, FAKE, 2_654_208, 0, FAKE, FAKE, 1 << 20, None]

    def call(i, v):
        a = list(base)
        a[i] = v
        return g(*a)
    assert call(1, 9) == _lib.MOE_ESHAPE             # T > 8
    assert call(1, 0) == _lib.MOE_ESHAPE
    assert call(11, 3) == _lib.MOE_EUNSUPPORTED      # qfmt
    assert call(9, FAKE + 64) == _lib.MOE_EALIGN     # pool alignment
    assert call(10, 2_654_208 - 256) == _lib.MOE_EALIGN  # record too small
    assert call(10, 2_654_208 + 1) == _lib.MOE_EALIGN
    assert call(13, None) == _lib.MOE_EWORKSPACE
    assert call(14, 100) == _lib.MOE_EWORKSPACE
    assert call(7, None) == _lib.MOE_EINVAL          # slot table
    assert call(3, 700) == _lib.MOE_ESHAPE           # F % 128
    assert call(5, 17) == _lib.MOE_ESHAPE            # k > 16
    h = lib.moe_grouped_gemm_q
    gb = [FAKE, 8192, 2048, 768, FAKE, FAKE, 10, 512, FAKE, 0, FAKE, 2_654_208, 0, FAKE, FAKE, _lib.MOE_F16, FAKE, 0,
          None]
    assert h(*gb) == _lib.MOE_EWORKSPACE
    gb2 = list(gb); gb2[0] = FAKE + 2
    gb2[17] = 1 << 40
    assert h(*gb2) == _lib.MOE_EALIGN
    gb3 = list(gb); gb3[7] = 4096
    assert h(*gb3) == _lib.MOE_ESHAPE
    gb4 = list(gb); gb4[15] = _lib.MOE_BF16          # output rows: fp32 or fp16 only
    assert h(*gb4) == _lib.MOE_EUNSUPPORTED
    gb5 = list(gb); gb5[1] = 1 << 20                 # fp16 copies past 32-bit byte offsets
    assert h(*gb5) == _lib.MOE_ESHAPE
    for i in (13, 14):                               # y_perm, y_shared: 16-byte vector stores
        gb6 = list(gb); gb6[i] = FAKE + 8
        gb6[17] = 1 << 40
        assert h(*gb6) == _lib.MOE_EALIGN


def test_permute_combine_usage_reject(lib):
    assert lib.moe_permute(FAKE, 10, 2, 0, FAKE, FAKE, FAKE, FAKE, None, 0, 0, None, FAKE, 1 << 20, None) == _lib.MOE_ESHAPE
    assert lib.moe_permute(FAKE, 10, 2, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 256, None, FAKE, 1 << 20, None) == _lib.MOE_EINVAL
    assert lib.moe_permute(FAKE, 1000, 10, 512, FAKE, FAKE, FAKE, FAKE, None, 0, 0, None, FAKE, 8, None) == _lib.MOE_EWORKSPACE
    F32, F16 = _lib.MOE_F32, _lib.MOE_F16
    assert lib.moe_combine(FAKE, F32, FAKE, None, FAKE, None, 4, 2, 256, FAKE, None) == _lib.MOE_EINVAL
    assert lib.moe_combine(FAKE, F16, None, None, FAKE, None, 4, 2, 254, FAKE, None) == _lib.MOE_ESHAPE
    assert lib.moe_combine(FAKE + 4, F32, None, None, FAKE, None, 4, 2, 256, FAKE, None) == _lib.MOE_EALIGN
    assert lib.moe_combine(FAKE, _lib.MOE_BF16, None, None, FAKE, None, 4, 2, 256, FAKE, None) == _lib.MOE_EUNSUPPORTED
    u = lib.moe_usage_update
    assert u(FAKE, 1, 10, 48, 48, 512, ctypes.c_float(0.99), 0, 4, 96, FAKE, FAKE, FAKE, None) == _lib.MOE_EINVAL
    assert u(FAKE, 1, 10, 0, 200, 512, ctypes.c_float(0.99), 0, 4, 96, FAKE, FAKE, FAKE, None) == _lib.MOE_ESHAPE
    assert u(FAKE, 1, 10, 0, 48, 512, ctypes.c_float(0.99), 0, 4, 2000, FAKE, FAKE, FAKE, None) == _lib.MOE_ESHAPE
    assert u(FAKE, 1, 10, 0, 48, 512, ctypes.c_float(float("nan")), 0, 4, 96, FAKE, FAKE, FAKE, None) == _lib.MOE_EINVAL
    assert u(FAKE, 1, 10, 0, 48, 512, ctypes.c_float(0.99), 0, 0, 96, FAKE, FAKE, FAKE, None) == _lib.MOE_EINVAL


def test_decode_stack_rejects(lib):
    f = lib.moe_decode_stack
    a = [FAKE, 1, 2048, 768, 512, 10, 48, FAKE, None, FAKE, FAKE, 2_654_208, 0, FAKE + 256, None, None, None, FAKE,
         1024, None]
    b = list(a); b[13] = FAKE
    assert f(*b) == _lib.MOE_EINVAL                   # x_out aliases x_in
    b = list(a); b[6] = 0
    assert f(*b) == _lib.MOE_ESHAPE
    assert f(*a) == _lib.MOE_EWORKSPACE               # 1 KiB is too small


def test_tier_rejects(lib):
    """Host-side validation of the hot-tier calls (no launch happens)."""
    fill = lib.moe_tier_fill
    a = [FAKE, 48, 512, 4096, FAKE, FAKE, FAKE, FAKE, 2_654_208, FAKE, FAKE, None]
    b = list(a); b[3] = 0
    assert fill(*b) == _lib.MOE_ESHAPE                # n_hot < 1
    b = list(a); b[3] = 48 * 512 + 1
    assert fill(*b) == _lib.MOE_ESHAPE                # n_hot > L*E
    b = list(a); b[1] = 200
    assert fill(*b) == _lib.MOE_ESHAPE                # L*E > 65536
    b = list(a); b[8] = 2_654_208 + 16
    assert fill(*b) == _lib.MOE_EALIGN                # record bytes not a multiple of 256
    b = list(a); b[7] = FAKE + 16
    assert fill(*b) == _lib.MOE_EALIGN                # pool not 256-byte aligned
    b = list(a); b[6] = None
    assert fill(*b) == _lib.MOE_EINVAL
    reb = lib.moe_tier_rebalance
    r = [FAKE, 48, 512, 4096, 96, FAKE, FAKE, FAKE, FAKE, 2_654_208, FAKE, FAKE, None]
    b = list(r); b[4] = 2000
    assert reb(*b) == _lib.MOE_ESHAPE                 # max_swaps > 1024
    b = list(r); b[4] = -1
    assert reb(*b) == _lib.MOE_ESHAPE                 # max_swaps < 0
    b = list(r); b[3] = 0
    assert reb(*b) == _lib.MOE_ESHAPE                 # n_hot < 1
    b = list(r); b[11] = None
    assert reb(*b) == _lib.MOE_EINVAL                 # n_swaps missing


def test_usage_update_stack_rejects(lib):
    u = lib.moe_usage_update_stack
    a = [FAKE, 1, 10, 48, 512, ctypes.c_float(0.99), 0, 4, 96, FAKE, FAKE, FAKE, None]
    b = list(a); b[3] = 200
    assert u(*b) == _lib.MOE_ESHAPE                   # L*E > 65536
    b = list(a); b[8] = 2000
    assert u(*b) == _lib.MOE_ESHAPE                   # top_n > 1024
    b = list(a); b[7] = 0
    assert u(*b) == _lib.MOE_EINVAL                   # rerank_every < 1
    b = list(a); b[9] = None
    assert u(*b) == _lib.MOE_EINVAL                   # hits_ws missing


# ---------------------------------------------------------------- host-side index checks

def _i32(a):
    import numpy as np
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.c_void_p)


def test_validate_routing(lib):
    good, p = _i32([[3, 0, 7], [1, 2, 5]])
    assert lib.moe_validate_routing(p, 2, 3, 8) == _lib.MOE_OK
    assert lib.moe_validate_routing(p, 2, 3, 7) == _lib.MOE_EINVAL and "topk_idx[0][2] = 7" in _err(lib)
    dup, pd = _i32([[3, 0, 7], [1, 5, 5]])
    assert lib.moe_validate_routing(pd, 2, 3, 8) == _lib.MOE_EINVAL and "twice" in _err(lib)
    neg, pn = _i32([[3, -1, 7]])
    assert lib.moe_validate_routing(pn, 1, 3, 8) == _lib.MOE_EINVAL
    assert lib.moe_validate_routing(None, 0, 3, 8) == _lib.MOE_OK
    assert lib.moe_validate_routing(p, 2, 9, 8) == _lib.MOE_ESHAPE  # k > E


def test_validate_slot_table(lib):
    S, p = _i32([[0, 5, 2], [4, 1, 3]])
    assert lib.moe_validate_slot_table(p, 2, 2, 6) == _lib.MOE_OK
    assert lib.moe_validate_slot_table(p, 2, 2, 5) == _lib.MOE_EINVAL and "slot_table[0][1] = 5" in _err(lib)
    assert lib.moe_validate_slot_table(None, 2, 2, 6) == _lib.MOE_EINVAL


def test_validate_rows(lib):
    import numpy as np
    import oracle as O
    idx = np.array([[2, 0], [0, 1], [2, 1]])
    counts, offsets, row_src, inv_row = O.permute(idx, 4)
    o, po = _i32(offsets)
    r, pr = _i32(row_src)
    i, pi = _i32(inv_row)
    assert lib.moe_validate_rows(po, pr, pi, 3, 2, 4) == _lib.MOE_OK
    assert lib.moe_validate_rows(po, pr, None, 3, 2, 4) == _lib.MOE_OK
    bad_o, pbo = _i32([0, 2, 1, 6, 6])
    assert lib.moe_validate_rows(pbo, pr, pi, 3, 2, 4) == _lib.MOE_EINVAL and "offsets[2]" in _err(lib)
    short, pso = _i32([0, 2, 4, 5, 5])
    assert lib.moe_validate_rows(pso, pr, pi, 3, 2, 4) == _lib.MOE_EINVAL
    rep = r.copy()
    rep[1] = rep[0]
    _, prep = _i32(rep)
    assert lib.moe_validate_rows(po, prep, None, 3, 2, 4) == _lib.MOE_EINVAL and "repeats" in _err(lib)
    wrong_inv = i.copy()
    wrong_inv[[0, 1]] = wrong_inv[[1, 0]]
    _, pwi = _i32(wrong_inv)
    assert lib.moe_validate_rows(po, pr, pwi, 3, 2, 4) == _lib.MOE_EINVAL and "inv_row" in _err(lib)
    oob = r.copy()
    oob[3] = 6
    _, poob = _i32(oob)
    assert lib.moe_validate_rows(po, poob, None, 3, 2, 4) == _lib.MOE_EINVAL


def test_binding_validates_before_launching(monkeypatch):
    """MOE_VALIDATE=1: the binding runs the host checks on a call's index
    arrays (CPU tensors here) and raises before anything reaches the GPU."""
    import torch
    from routed_expert_ffn_moe_amd import ops
    monkeypatch.setenv("MOE_VALIDATE", "1")
    with pytest.raises(ops.MoeError, match="outside"):
        ops.validate_routing(torch.tensor([[0, 16]]), 16)
    with pytest.raises(ops.MoeError, match="twice"):
        ops.validate_routing(torch.tensor([[3, 3]]), 16)
    with pytest.raises(ops.MoeError, match="slot_table"):
        ops.validate_slot_table(torch.tensor([[0, 1, 9]]), 9)
    ops.validate_rows(torch.tensor([0, 1, 2]), torch.tensor([1, 0]), 1, 2)
    with pytest.raises(ops.MoeError):
        ops.validate_rows(torch.tensor([0, 1, 2]), torch.tensor([1, 1]), 1, 2)


def test_noalloc_checks_arguments_before_any_device_call(lib):
    """The no-alloc decode step validates its arguments like moe_decode_stack
    before it looks up a device; with valid ones and no GPU it stops at the
    device lookup with MOE_EHIP."""
    R = lib.moe_record_bytes(0, 2048, 768)
    args = [FAKE, 1, 2048, 768, 512, 10, 48, FAKE, None, FAKE, FAKE, R, 0, FAKE + 0x1000, None, None, None, None]
    bad = list(args)
    bad[1] = 9  # T > MOE_MAX_DECODE_T
    assert lib.moe_decode_stack_noalloc(*bad) == _lib.MOE_ESHAPE
    bad = list(args)
    bad[13] = FAKE  # x_out aliases x_in
    assert lib.moe_decode_stack_noalloc(*bad) == _lib.MOE_EINVAL
    assert lib.moe_decode_stack_noalloc(*args) == _lib.MOE_EHIP and "no-alloc" in _err(lib)


def test_rmsnorm_rejects(lib):
    assert lib.moe_rmsnorm(FAKE, 4, 256, 1e-6, FAKE + 0x1000, 7, None) == _lib.MOE_EUNSUPPORTED
    assert lib.moe_rmsnorm(FAKE, -1, 256, 1e-6, FAKE + 0x1000, 0, None) == _lib.MOE_ESHAPE
    assert lib.moe_rmsnorm(FAKE, 4, 256, -1.0, FAKE + 0x1000, 0, None) == _lib.MOE_EINVAL
    assert lib.moe_rmsnorm(FAKE, 4, 256, 1e-6, FAKE, 1, None) == _lib.MOE_EINVAL  # aliasing
    assert lib.moe_rmsnorm(None, 0, 256, 1e-6, None, 1, None) == _lib.MOE_OK      # nothing to do


def test_probe_header_symbols_are_exported(lib):
    names = declared_functions(PROBES)
    assert len(names) == 8, names
    for n in names:
        assert hasattr(lib, n) and n in _lib.SIGNATURES, n
    assert lib.moe_probe_stream_read(None, 16, FAKE, None) == _lib.MOE_EINVAL
    assert lib.moe_probe_stream_read(FAKE + 4, 16, FAKE, None) == _lib.MOE_EALIGN
    assert lib.moe_probe_mfma(0, FAKE, None) == _lib.MOE_EINVAL
    assert lib.moe_probe_exchange(3, 10, FAKE, 1 << 30, FAKE, FAKE, None) == _lib.MOE_EINVAL
    assert lib.moe_probe_exchange(0, 0, FAKE, 1 << 30, FAKE, FAKE, None) == _lib.MOE_EINVAL
    assert lib.moe_probe_exchange(0, 10, FAKE, 8, FAKE, FAKE, None) == _lib.MOE_EWORKSPACE
