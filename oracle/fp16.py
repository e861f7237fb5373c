"""IEEE-754 binary16 codec of the oracle (NumPy integer arithmetic only; test
infrastructure).

A binary16 value is carried as its 16-bit pattern in a ``numpy.uint16`` array
(1 sign bit, 5 exponent bits with bias 15, 10 fraction bits).  The pages use
fp16 for tensor-parallel activations and name no rounding rule, so the
IEEE-754 default is the reading taken:

* widen: exact -- every binary16 value, subnormals included, is a binary32
  value.
* narrow: round to nearest, ties to even, from the binary32 pattern.  Values
  whose magnitude rounds to 2^16 or more become +-inf.  Results below 2^-14
  are binary16 subnormals (multiples of 2^-24), rounded the same way; a
  binary32 subnormal is far below half of 2^-24 and gives +-0.  A NaN keeps
  its sign and its top 9 payload bits and gets the quiet bit (0x0200), so it
  cannot turn into an infinity.
"""

import numpy as np


def widen(h):
    """binary16 bit patterns (uint16) -> float32 values, exactly."""
    h = np.asarray(h, dtype=np.uint16).astype(np.int64)
    sign = np.where(h & 0x8000, -1.0, 1.0)
    e = (h >> 10) & 0x1F
    m = (h & 0x3FF).astype(np.float64)
    normal = sign * (1.0 + m / 1024.0) * np.exp2(e.astype(np.float64) - 15.0)
    sub = sign * m * 2.0 ** -24
    out = np.where(e == 0, sub, np.where(e == 31, np.where(m == 0, sign * np.inf, np.nan), normal))
    # float64 -> float32 is exact for every binary16 value; restore NaN payloads bit for bit
    res = out.astype(np.float32)
    nan = (e == 31) & ((h & 0x3FF) != 0)
    bits = ((h & 0x8000) << 16) | 0x7F800000 | ((h & 0x3FF) << 13)
    res = np.where(nan, bits.astype(np.uint32).view(np.float32), res)
    return res.astype(np.float32)


def _round_shift(v, shift):
    """v >> shift, rounded to nearest with ties to even (v, shift int64 arrays, shift >= 1)."""
    q = v >> shift
    rem = v & ((np.int64(1) << shift) - 1)
    half = np.int64(1) << (shift - 1)
    up = (rem > half) | ((rem == half) & ((q & 1) == 1))
    return q + up.astype(np.int64)


def narrow(f):
    """float32 values -> binary16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.int64)
    sign = (u >> 16) & 0x8000
    a = u & 0x7FFFFFFF
    exp32 = a >> 23
    frac32 = a & 0x7FFFFF
    sig = frac32 | 0x800000  # 24-bit significand of a normal binary32 value
    # normal binary16 range: unbiased exponent >= -14, i.e. exp32 >= 113
    e16 = exp32 - 112
    normal = ((np.maximum(e16, 0) << 10) | (frac32 >> 13))
    rem = frac32 & 0x1FFF
    up = (rem > 0x1000) | ((rem == 0x1000) & ((normal & 1) == 1))
    normal = normal + up.astype(np.int64)  # a carry moves into the exponent; 0x7C00 is inf
    # subnormal binary16: value = sig * 2^(exp32 - 150) = q * 2^-24, q = sig >> (126 - exp32)
    shift = np.clip(126 - exp32, 1, 62)
    sub = np.where(exp32 >= 101, _round_shift(sig, shift), 0)  # below 2^-25: rounds to 0
    res = np.where(exp32 >= 113, normal, sub)
    res = np.where(res >= 0x7C00, 0x7C00, res)  # overflow -> inf
    res = np.where(a == 0x7F800000, 0x7C00, res)
    nan = a > 0x7F800000
    res = np.where(nan, 0x7C00 | 0x0200 | (frac32 >> 13), res)
    return (sign | res).astype(np.uint16)
