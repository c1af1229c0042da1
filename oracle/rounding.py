"""Rounding of real values to bfloat16 in the three modes the benchmark page reports
(7minutos.es article on MoonMath AI's kernel, section "Punto de referencia": RTNE
rounds to the nearest value with ties to even, RTNA to the nearest with ties away
from zero, RTZ truncates toward zero). TEST INFRASTRUCTURE ONLY.

bfloat16 has 1 sign bit, 8 exponent bits (bias 127) and 7 fraction bits: in each
binade [2^e, 2^(e+1)) its values are 2^e * (1 + k / 128), k = 0..127; below 2^-126
the subnormals are k * 2^-133. Values beyond the largest finite one round to
infinity where the mode's rule sends them there (RTZ never does).

The functions work on float64 inputs with exact integer arithmetic on the scaled
value (math.frexp / ldexp are exact), element by element.
"""
import math

import numpy as np

MODES = ("rtne", "rtna", "rtz")
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127          # largest finite bfloat16
_MIN_NORMAL_EXP = -126
_FRAC_BITS = 7


def round_bf16_scalar(x: float, mode: str) -> float:
    """The bfloat16 value that `x` rounds to under `mode`, as a float."""
    if mode not in MODES:
        raise ValueError(f"mode must be one of {MODES}")
    if math.isnan(x) or math.isinf(x) or x == 0.0:
        return x
    sign = -1.0 if x < 0 else 1.0
    a = abs(x)
    m, e = math.frexp(a)                # a = m * 2^e, 0.5 <= m < 1
    e -= 1                              # a = (2m) * 2^e, 1 <= 2m < 2
    e = max(e, _MIN_NORMAL_EXP)         # subnormals share the spacing of the smallest binade
    ulp_exp = e - _FRAC_BITS            # spacing of bfloat16 values around a
    scaled = math.ldexp(a, -ulp_exp)    # a / ulp, exact
    lo = math.floor(scaled)
    frac = scaled - lo                  # exact: scaled has few significant bits
    if mode == "rtz":
        k = lo
    elif frac > 0.5:
        k = lo + 1
    elif frac < 0.5:
        k = lo
    elif mode == "rtna":
        k = lo + 1
    else:                               # rtne: tie to the even neighbour
        k = lo + (lo & 1)
    r = math.ldexp(float(k), ulp_exp)
    if r > BF16_MAX:
        r = math.inf
    return sign * r


def round_bf16(x, mode: str) -> np.ndarray:
    """Element-wise round_bf16_scalar over an array of float64 values."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.float64)
    flat_in, flat_out = a.reshape(-1), out.reshape(-1)    # views of contiguous arrays
    for i in range(flat_in.size):
        flat_out[i] = round_bf16_scalar(float(flat_in[i]), mode)
    return out
