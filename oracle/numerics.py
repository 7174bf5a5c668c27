"""Scalar helpers of the oracle: bf16 rounding, SiLU, first-index argmax (fp64).

Test infrastructure only (see ``oracle/__init__``).
"""
import numpy as np


def round_bf16(x):
    """Round to the nearest bfloat16 value (ties to even), returned as float64.

    The pages fix no precision; the product path stores intermediate tensors in
    bf16 at fixed points and this emulates that storage step.  The value is
    first rounded to float32 (nearest-even), then the low 16 bits of the
    float32 pattern are rounded away with ties to even.
    """
    a = np.asarray(x, dtype=np.float64).astype(np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = (bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def silu(x):
    """SiLU(x) = x * sigmoid(x), as used inside the Medusa head residual block."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def argmax_first(x, axis=-1):
    """Index of the largest value; among equal values the lowest index wins.

    This is the tie rule of ``torch.argmax`` on the pages' code.
    """
    return np.argmax(np.asarray(x), axis=axis)
