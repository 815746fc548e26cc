"""CPU oracle for the Hadamard-rotated 1-bit matrix-vector product.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the tests, the smoke check and the CPU-baseline
leg of the benchmark do.  It shares no code with the HIP library.
"""
from .pq1_oracle import *  # noqa: F401,F403
