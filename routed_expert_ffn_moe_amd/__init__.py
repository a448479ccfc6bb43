"""MI355X (gfx950) routed-expert MoE-FFN layer: Python binding of libmoe.so.

The layer's kernels are hand-written HIP in csrc/ behind the C ABI of
include/moe.h; this package only loads the library and marshals tensors.
"""
from .ops import *  # noqa: F401,F403
from ._lib import MoeError, MoeNotBuilt, load  # noqa: F401
