"""CPU oracle for the MoE expert layer: TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 numpy. It shares no code with the HIP library and imports
nothing from it. Only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import this package; the product path never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
