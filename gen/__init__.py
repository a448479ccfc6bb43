"""Seeded synthetic inputs for the MoE-FFN layer (x, router, bias, quantised
expert records, pool and slot table).

This package is shared by the oracle side and the HIP side.  It holds none of
the layer's arithmetic: it draws random numbers, encodes weights into the
record byte format of include/moe.h and places records into a pool.
"""
from .inputs import *  # noqa: F401,F403
