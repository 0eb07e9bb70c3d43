"""The OCP FP8 E4M3 encoding: code values and round-to-nearest encoding.

TEST INFRASTRUCTURE ONLY (part of the CPU oracle; see ``oracle/fp8.py`` for
the readings).  E4M3: sign, 4 exponent bits with bias 7, 3 mantissa bits,
subnormals at exponent field 0, no infinities, S.1111.111 is NaN; the largest
finite magnitude is 448.  Imports nothing from the rest of the oracle.
"""
from __future__ import annotations

import numpy as np

E4M3 = "e4m3"
E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def e4m3_value(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8) as float64; NaN for S.1111.111.

    Exponent field e, mantissa m: e = 0 gives the subnormal m * 2^-9, else
    (1 + m/8) * 2^(e - 7) = (8 + m) * 2^(e - 10).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7 == 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2((e - 10).astype(np.float64)))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# the finite non-negative codes 0x00 .. 0x7E in increasing order of value
_POS_VALUES = e4m3_value(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x) -> np.ndarray:
    """E4M3 code of each float32 value: nearest, ties to the even code,
    saturating at +-448, NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64))
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    # neighbours T[hi-1] < a <= T[hi] among the finite magnitudes
    hi = np.clip(np.searchsorted(_POS_VALUES, np.minimum(a, E4M3_MAX), side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    out = (sign | code).astype(np.int64)
    out = np.where(np.isnan(x), E4M3_NAN, out)
    return out.astype(np.uint8)
