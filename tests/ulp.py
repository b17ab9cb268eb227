"""Distance in bf16 units in the last place between raw bit patterns (+0 and -0 are equal)."""
import numpy as np


def ordinal(bits):
    b = np.asarray(bits).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_diff(a, b):
    return np.abs(ordinal(a) - ordinal(b))


def is_nan(bits):
    b = np.asarray(bits).astype(np.int32)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)
