"""Seeded synthetic inputs shared by the product path, the tests and the oracle.

This package holds input generation only -- random tensors with the shapes and
value distributions of the workloads, tree configurations (rank-path choice
lists), and bfloat16 packing of generated values.  It holds none of the Medusa
arithmetic: no heads, no tree buffers, no attention, no acceptance.
"""
from .gen import *  # noqa: F401,F403
from .trees import *  # noqa: F401,F403
