"""ctypes loader of libmoe.so and its C signatures (include/moe.h)."""
import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")
HEADER = os.path.join(HERE, "..", "include", "moe.h")

# constants of include/moe.h
MOE_OK, MOE_EINVAL, MOE_ESHAPE, MOE_EALIGN, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4, -5, -6
MOE_F32, MOE_BF16, MOE_F16 = 0, 1, 2
MOE_Q4_B32, MOE_Q2_B16 = 0, 1
(MOE_OP_ROUTE_TOPK, MOE_OP_PERMUTE, MOE_OP_EXPERT_GEMV_Q, MOE_OP_GROUPED_GEMM_Q, MOE_OP_COMBINE,
 MOE_OP_USAGE_UPDATE, MOE_OP_DECODE_STACK) = range(7)
MOE_MAX_E, MOE_MAX_K, MOE_MAX_DECODE_T = 1024, 16, 8
MOE_NOALLOC_WS_BYTES = 24 << 20

_vp, _i, _i64, _sz, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float

SIGNATURES = {
    "moe_abi_version": (_i, []),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_record_bytes": (_i64, [_i, _i, _i]),
    "moe_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "moe_route_topk": (_i, [_vp, _i, _i, _i, _vp, _vp, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_permute": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _sz, _vp]),
    "moe_expert_gemv_q": (_i, [_vp, _i, _i, _i, _vp, _i, _i, _vp, _i, _vp, _i64, _i, _vp, _vp, _sz, _vp]),
    "moe_grouped_gemm_q": (_i, [_vp, _i, _i, _i, _vp, _vp, _i, _i, _vp, _i, _vp, _i64, _i, _vp, _vp, _i, _vp, _sz,
                                _vp]),
    "moe_combine": (_i, [_vp, _i, _vp, _vp, _vp, _vp, _i, _i, _i, _vp, _vp]),
    "moe_usage_update": (_i, [_vp, _i, _i, _i, _i, _i, _f, _i64, _i, _i, _vp, _vp, _vp, _vp]),
    "moe_usage_update_stack": (_i, [_vp, _i, _i, _i, _i, _f, _i64, _i, _i, _vp, _vp, _vp, _vp]),
    "moe_tier_fill": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp]),
    "moe_tier_rebalance": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp]),
    "moe_decode_stack": (_i, [_vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i64, _i, _vp, _vp, _vp, _vp, _vp,
                              _sz, _vp]),
    "moe_decode_stack_noalloc": (_i, [_vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _i64, _i, _vp, _vp, _vp,
                                      _vp, _vp]),
    "moe_rmsnorm": (_i, [_vp, _i, _i, _f, _vp, _i, _vp]),
    # measurement probes (include/moe_probes.h)
    "moe_probe_stream_read": (_i, [_vp, _sz, _vp, _vp]),
    "moe_probe_stream_read_blocks": (_i, []),
    "moe_probe_mfma": (_i, [_i, _vp, _vp]),
    "moe_probe_mfma_blocks": (_i, []),
    "moe_probe_mfma_flops": (ctypes.c_double, [_i]),
    "moe_probe_exchange": (_i, [_i, _i, _vp, _sz, _vp, _vp, _vp]),
    "moe_probe_exchange_blocks": (_i, []),
    "moe_probe_exchange_ws_bytes": (_sz, []),
    "moe_validate_routing": (_i, [_vp, _i, _i, _i]),
    "moe_validate_slot_table": (_i, [_vp, _i, _i, _i64]),
    "moe_validate_rows": (_i, [_vp, _vp, _vp, _i, _i, _i]),
}


class MoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libmoe error {code}: {msg}")
        self.code = code


class MoeNotBuilt(RuntimeError):
    pass


_lock = threading.Lock()
_lib = None


def load(build_if_missing=True):
    """The loaded libmoe.so.  Builds it first only when no library exists."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            if not build_if_missing:
                raise MoeNotBuilt(f"{LIB_PATH} is missing; run routed_expert_ffn_moe_amd.build")
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def check(rc):
    if rc != MOE_OK:
        raise MoeError(rc, load().moe_last_error().decode(errors="replace"))
    return rc
