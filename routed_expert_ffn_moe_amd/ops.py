"""Python binding of libmoe: one function per C entry point, same names.

Only argument marshalling happens here: tensors are checked for device,
dtype and contiguity, missing outputs and workspaces are allocated with
torch (device memory is torch's job), and the C function is called with the
raw device pointers and torch's current HIP stream.  Every step of the layer
runs in the library's kernels; nothing here computes.
"""
import ctypes
import os

import torch

from . import _lib
from ._lib import (MOE_BF16, MOE_F16, MOE_F32, MOE_OP_DECODE_STACK, MOE_OP_EXPERT_GEMV_Q, MOE_OP_GROUPED_GEMM_Q,
                   MOE_OP_PERMUTE, MOE_OP_ROUTE_TOPK, MOE_Q2_B16, MOE_Q4_B32, MoeError, check)

__all__ = [
    "moe_abi_version", "moe_record_bytes", "moe_workspace_size", "workspace", "moe_route_topk", "moe_permute",
    "moe_expert_gemv_q", "moe_grouped_gemm_q", "moe_combine", "moe_usage_update", "moe_decode_stack",
    "moe_tier_fill", "moe_tier_rebalance", "moe_usage_update_stack", "moe_decode_stack_noalloc", "moe_rmsnorm",
    "MOE_Q4_B32", "MOE_Q2_B16", "MoeError", "MOE_OP_ROUTE_TOPK", "MOE_OP_PERMUTE", "MOE_OP_EXPERT_GEMV_Q",
    "MOE_OP_GROUPED_GEMM_Q", "MOE_OP_DECODE_STACK", "validate_routing", "validate_slot_table", "validate_rows",
]


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("libmoe takes device tensors only")
            if not t.is_contiguous():
                raise ValueError("libmoe takes contiguous tensors only")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _x_dtype(x):
    if x.dtype == torch.float32:
        return MOE_F32
    if x.dtype in (torch.bfloat16, torch.int16):  # bf16 values or their bit patterns
        return MOE_BF16
    raise ValueError(f"unsupported activation dtype {x.dtype}")


def _half_bits(t):
    if t.dtype not in (torch.bfloat16, torch.float16, torch.int16):
        raise ValueError(f"expected 16-bit tensor, got {t.dtype}")
    return t


# ---------------------------------------------------------------- index checks
# With MOE_VALIDATE=1 every call below first copies its index arrays to the
# host and runs the library's host-side checks on them (a debugging aid: it
# synchronises the stream).

def _validating():
    return os.environ.get("MOE_VALIDATE") == "1"


def _host_i32(t):
    return t.detach().to(device="cpu", dtype=torch.int32).contiguous()


def validate_routing(topk_idx, E):
    """topk_idx [T][k]: ids in [0, E), distinct per token (host check)."""
    h = _host_i32(topk_idx)
    T, k = h.shape
    check(_lib.load().moe_validate_routing(_p(h), T, k, E))


def validate_slot_table(slot_table, n_slots):
    """slot_table [L][E+1]: every slot in [0, n_slots) (host check)."""
    h = _host_i32(slot_table)
    L, E1 = h.shape
    check(_lib.load().moe_validate_slot_table(_p(h), L, E1 - 1, int(n_slots)))


def validate_rows(offsets, row_src, T, k, inv_row=None):
    """offsets [E+1] / row_src / inv_row [T*k] as moe_permute defines them (host check)."""
    ho, hr = _host_i32(offsets), _host_i32(row_src)
    hi = None if inv_row is None else _host_i32(inv_row)
    check(_lib.load().moe_validate_rows(_p(ho), _p(hr), _p(hi), T, k, ho.numel() - 1))


def _pool_slots(pool, record_bytes):
    return pool.numel() * pool.element_size() // record_bytes


def moe_abi_version():
    return _lib.load().moe_abi_version()


def moe_record_bytes(qfmt, H, F):
    return _lib.load().moe_record_bytes(qfmt, H, F)


def moe_workspace_size(op, T=0, k=0, E=0, H=0, F=0, qfmt=0):
    return _lib.load().moe_workspace_size(op, T, k, E, H, F, qfmt)


def workspace(op, device, T=0, k=0, E=0, H=0, F=0, qfmt=0):
    """Scratch for entry point `op`.  The decode-stack workspace is zero-filled
    (its header then starts a fresh tag count); the others need no contents."""
    n = max(moe_workspace_size(op, T, k, E, H, F, qfmt), 256)
    if op == MOE_OP_DECODE_STACK:
        return torch.zeros(n, dtype=torch.uint8, device=device)
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_route_topk(x, w_router, bias, k, topk_idx=None, topk_w=None, logits_out=None, ws=None, stream=None):
    """x [T][H] fp32/bf16, w_router bf16 [E][H], bias fp32 [E] or None."""
    T, H = x.shape
    E = w_router.shape[0]
    _half_bits(w_router)
    dev = x.device
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    if logits_out is None and ws is None:
        ws = workspace(MOE_OP_ROUTE_TOPK, dev, T=T, E=E)
    _dev(x, w_router, bias, topk_idx, topk_w, logits_out, ws)
    check(_lib.load().moe_route_topk(_p(x), _x_dtype(x), T, H, _p(w_router), _p(bias), E, k, _p(topk_idx),
                                     _p(topk_w), _p(logits_out), _p(ws), 0 if ws is None else ws.numel(),
                                     _stream(stream)))
    return topk_idx, topk_w


def moe_permute(topk_idx, E, counts=None, offsets=None, row_src=None, inv_row=None, x=None, x_perm=None, ws=None,
                stream=None):
    T, k = topk_idx.shape
    dev = topk_idx.device
    counts = torch.empty(E, dtype=torch.int32, device=dev) if counts is None else counts
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    row_src = torch.empty(T * k, dtype=torch.int32, device=dev) if row_src is None else row_src
    inv_row = torch.empty(T * k, dtype=torch.int32, device=dev) if inv_row is None else inv_row
    if x is not None and x_perm is None:
        x_perm = torch.empty((T * k, x.shape[1]), dtype=x.dtype, device=dev)
    ws = workspace(MOE_OP_PERMUTE, dev, T=T, k=k, E=E) if ws is None else ws
    _dev(topk_idx, counts, offsets, row_src, inv_row, x, x_perm, ws)
    if _validating():
        validate_routing(topk_idx, E)
    H = 0 if x is None else x.shape[1]
    xd = 0 if x is None else _x_dtype(x)
    check(_lib.load().moe_permute(_p(topk_idx), T, k, E, _p(counts), _p(offsets), _p(row_src), _p(inv_row), _p(x),
                                  xd, H, _p(x_perm), _p(ws), ws.numel(), _stream(stream)))
    return counts, offsets, row_src, inv_row, x_perm


def moe_expert_gemv_q(x, topk_idx, E, F, slot_table, layer, pool, record_bytes, qfmt, y_parts=None, ws=None,
                      stream=None):
    """x fp32 [T][H]; returns y_parts fp32 [T][k+1][H]."""
    T, H = x.shape
    k = topk_idx.shape[1]
    dev = x.device
    if y_parts is None:
        y_parts = torch.empty((T, k + 1, H), dtype=torch.float32, device=dev)
    ws = workspace(MOE_OP_EXPERT_GEMV_Q, dev, T, k, E, H, F, qfmt) if ws is None else ws
    _dev(x, topk_idx, slot_table, pool, y_parts, ws)
    if _validating():
        validate_routing(topk_idx, E)
        validate_slot_table(slot_table, _pool_slots(pool, record_bytes))
    check(_lib.load().moe_expert_gemv_q(_p(x), T, H, F, _p(topk_idx), k, E, _p(slot_table), layer, _p(pool),
                                        record_bytes, qfmt, _p(y_parts), _p(ws), ws.numel(), _stream(stream)))
    return y_parts


def _rows_dtype(t):
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.float16:
        return MOE_F16
    raise TypeError(f"expert output rows must be float32 or float16, got {t.dtype}")


def moe_grouped_gemm_q(x, row_src, offsets, k, E, F, slot_table, layer, pool, record_bytes, qfmt, y_perm=None,
                       y_shared=None, ws=None, stream=None, y_dtype=torch.float16):
    """x bf16 [T][H]; returns (y_perm [T*k][H], y_shared [T][H]) in y_dtype
    (float16 by default, or float32; given output tensors set it)."""
    T, H = x.shape
    dev = x.device
    _half_bits(x)
    if y_perm is not None:
        y_dtype = y_perm.dtype
    y_perm = torch.empty((T * k, H), dtype=y_dtype, device=dev) if y_perm is None else y_perm
    y_shared = torch.empty((T, H), dtype=y_dtype, device=dev) if y_shared is None else y_shared
    yd = _rows_dtype(y_perm)
    if y_shared.dtype != y_perm.dtype:
        raise TypeError("y_perm and y_shared must have the same dtype")
    ws = workspace(MOE_OP_GROUPED_GEMM_Q, dev, T, k, E, H, F, qfmt) if ws is None else ws
    _dev(x, row_src, offsets, slot_table, pool, y_perm, y_shared, ws)
    if _validating():
        validate_rows(offsets, row_src, T, k)
        validate_slot_table(slot_table, _pool_slots(pool, record_bytes))
    check(_lib.load().moe_grouped_gemm_q(_p(x), T, H, F, _p(row_src), _p(offsets), k, E, _p(slot_table), layer,
                                         _p(pool), record_bytes, qfmt, _p(y_perm), _p(y_shared), yd, _p(ws),
                                         ws.numel(), _stream(stream)))
    return y_perm, y_shared


def moe_combine(y_rows, topk_w, inv_row=None, y_shared=None, residual=None, y_out=None, stream=None):
    """y_rows (and y_shared) float32 or float16; y_out float32 [T][H]."""
    T, k = topk_w.shape
    H = y_rows.shape[-1]
    rd = _rows_dtype(y_rows)
    if y_shared is not None and y_shared.dtype != y_rows.dtype:
        raise TypeError("y_rows and y_shared must have the same dtype")
    y_out = torch.empty((T, H), dtype=torch.float32, device=y_rows.device) if y_out is None else y_out
    _dev(y_rows, topk_w, inv_row, y_shared, residual, y_out)
    if _validating() and inv_row is not None:  # inv_row must be a permutation of the T*k rows
        n = T * k
        validate_rows(torch.tensor([0, n], dtype=torch.int32), inv_row, T, k)
    check(_lib.load().moe_combine(_p(y_rows), rd, _p(inv_row), _p(y_shared), _p(topk_w), _p(residual), T, k, H,
                                  _p(y_out), _stream(stream)))
    return y_out


def moe_usage_update(topk_idx, layer, L, E, decay, step, rerank_every, top_n, hits_ws, scores, top_out=None,
                     stream=None):
    T, k = topk_idx.shape
    _dev(topk_idx, hits_ws, scores, top_out)
    if _validating():
        validate_routing(topk_idx, E)
    check(_lib.load().moe_usage_update(_p(topk_idx), T, k, layer, L, E, float(decay), int(step), rerank_every, top_n,
                                       _p(hits_ws), _p(scores), _p(top_out), _stream(stream)))
    return scores, top_out


def moe_tier_fill(scores, n_hot, home_table, slot_table, hot_owner, pool, record_bytes, swaps, n_swaps,
                  stream=None):
    """scores fp32 [L][E]; home_table / slot_table int32 [L][E+1]; hot_owner
    int32 [n_hot]; swaps int32 [>= n_hot][4]; n_swaps int32 [1]."""
    L, E = scores.shape
    _dev(scores, home_table, slot_table, hot_owner, pool, swaps, n_swaps)
    check(_lib.load().moe_tier_fill(_p(scores), L, E, n_hot, _p(home_table), _p(slot_table), _p(hot_owner), _p(pool),
                                    record_bytes, _p(swaps), _p(n_swaps), _stream(stream)))
    return slot_table, hot_owner


def moe_tier_rebalance(scores, n_hot, max_swaps, home_table, slot_table, hot_owner, pool, record_bytes, swaps,
                       n_swaps, stream=None):
    """scores fp32 [L][E]; swaps int32 [>= max_swaps][4]."""
    L, E = scores.shape
    _dev(scores, home_table, slot_table, hot_owner, pool, swaps, n_swaps)
    check(_lib.load().moe_tier_rebalance(_p(scores), L, E, n_hot, max_swaps, _p(home_table), _p(slot_table),
                                         _p(hot_owner), _p(pool), record_bytes, _p(swaps), _p(n_swaps),
                                         _stream(stream)))
    return slot_table, hot_owner


def moe_usage_update_stack(topk_idx, E, decay, step, rerank_every, top_n, hits_ws, scores, top_out=None,
                           stream=None):
    """topk_idx int32 [L][T][k]; hits_ws int32 [L][E]; scores fp32 [L][E]."""
    L, T, k = topk_idx.shape
    _dev(topk_idx, hits_ws, scores, top_out)
    if _validating():
        validate_routing(topk_idx.reshape(L * T, k), E)
    check(_lib.load().moe_usage_update_stack(_p(topk_idx), T, k, L, E, float(decay), int(step), rerank_every, top_n,
                                             _p(hits_ws), _p(scores), _p(top_out), _stream(stream)))
    return scores, top_out


def moe_decode_stack(x_in, F, E, k, w_router, bias, slot_table, pool, record_bytes, qfmt, x_out=None,
                     topk_idx_out=None, topk_w_out=None, x_hist=None, ws=None, stream=None):
    """x_in fp32 [T][H], w_router bf16 [L][E][H]; returns x_out fp32 [T][H]."""
    T, H = x_in.shape
    L = w_router.shape[0]
    dev = x_in.device
    x_out = torch.empty_like(x_in) if x_out is None else x_out
    ws = workspace(MOE_OP_DECODE_STACK, dev, T, k, E, H, F, qfmt) if ws is None else ws
    _dev(x_in, w_router, bias, slot_table, pool, x_out, topk_idx_out, topk_w_out, x_hist, ws)
    if _validating():
        validate_slot_table(slot_table, _pool_slots(pool, record_bytes))
    check(_lib.load().moe_decode_stack(_p(x_in), T, H, F, E, k, L, _p(w_router), _p(bias), _p(slot_table), _p(pool),
                                       record_bytes, qfmt, _p(x_out), _p(topk_idx_out), _p(topk_w_out), _p(x_hist),
                                       _p(ws), ws.numel(), _stream(stream)))
    return x_out


def moe_decode_stack_noalloc(x_in, F, E, k, w_router, bias, slot_table, pool, record_bytes, qfmt, x_out=None,
                             topk_idx_out=None, topk_w_out=None, x_hist=None, stream=None):
    """moe_decode_stack on the library's own per-device scratch (no workspace
    argument; the C entry point allocates nothing).  Pass x_out to keep this
    call free of torch allocations too."""
    T, H = x_in.shape
    L = w_router.shape[0]
    x_out = torch.empty_like(x_in) if x_out is None else x_out
    _dev(x_in, w_router, bias, slot_table, pool, x_out, topk_idx_out, topk_w_out, x_hist)
    if _validating():
        validate_slot_table(slot_table, _pool_slots(pool, record_bytes))
    check(_lib.load().moe_decode_stack_noalloc(_p(x_in), T, H, F, E, k, L, _p(w_router), _p(bias), _p(slot_table),
                                               _p(pool), record_bytes, qfmt, _p(x_out), _p(topk_idx_out),
                                               _p(topk_w_out), _p(x_hist), _stream(stream)))
    return x_out


def moe_rmsnorm(x, eps=1e-6, out=None, out_dtype=torch.bfloat16, stream=None):
    """x fp32 [T][H] -> x / rms(x) in fp32 or bf16 (the stack's pre-norm)."""
    T, H = x.shape
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=x.device)
    od = MOE_F32 if out.dtype == torch.float32 else MOE_BF16
    if od == MOE_BF16:
        _half_bits(out)
    _dev(x, out)
    check(_lib.load().moe_rmsnorm(_p(x), T, H, float(eps), _p(out), od, _stream(stream)))
    return out
