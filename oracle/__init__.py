"""CPU oracle for Sliding Tile Attention: test infrastructure only.

Only tests, the smoke check and the CPU-baseline leg of the benchmark may use
this package; the product path never imports it.
"""
from .sta_oracle import *  # noqa: F401,F403
