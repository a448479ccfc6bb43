"""CPU oracle of the routed-expert MoE-FFN layer -- TEST INFRASTRUCTURE.

Plain, slow, fp64 NumPy.  It shares no code with the HIP library and the
library never calls it: only the tests, the smoke check and the benchmark's
CPU-baseline leg import it.  See moe_oracle.py (the layer) and tier.py (the
hot tier of expert records) for what each function follows.
"""
from .moe_oracle import *  # noqa: F401,F403
