"""bfloat16 codec of the oracle (NumPy only; test infrastructure).

A bf16 value is carried as its 16-bit pattern in a ``numpy.uint16`` array:
the upper half of an IEEE-754 binary32.

* widen: exact -- the 16 bits become the upper half of a binary32 whose lower
  half is zero.
* narrow: round to nearest, ties to even (the IEEE-754 default; the pages fix
  no rounding mode, so the default is the reading taken).  The carry out of
  the mantissa into the exponent gives overflow to +-inf for free.  A NaN keeps
  its sign and top payload bits and is made quiet by setting the top mantissa
  bit, so that it can never turn into an infinity by truncation.
  Denormal binary32 inputs are rounded like any other value (no flush).
"""

import numpy as np


def widen(h):
    """bf16 bit patterns (uint16) -> float32 values, exactly."""
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def narrow(f):
    """float32 values -> bf16 bit patterns (uint16), round-to-nearest-even."""
    f = np.ascontiguousarray(f, dtype=np.float32)
    u = f.view(np.uint32)
    is_nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    quiet = (u >> np.uint32(16)) | np.uint32(0x0040)
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


def ulp_distance(a, b):
    """Distance in bf16 ulps between two bf16 bit-pattern arrays.

    The patterns are mapped to a monotone integer key (sign-magnitude to
    two's-complement order) with +0 and -0 on the same key, so adjacent
    representable values differ by 1.
    """

    def key(h):
        h = np.asarray(h, dtype=np.uint16).astype(np.int64)
        mag = h & 0x7FFF
        return np.where(h & 0x8000, -mag, mag)

    return np.abs(key(a) - key(b))
