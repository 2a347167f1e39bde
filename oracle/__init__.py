"""CPU oracle of the Hymba fused hybrid-head layer forward.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package.  The GPU library never calls it, and
it shares no code with the GPU library.
"""
from .hymba import *  # noqa: F401,F403
