"""Pure-Python attention for tiny inputs (no numpy arithmetic).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Computes, for one query row, s_j = tau * sum_c q_c k_jc over the visible keys,
then O = sum_j exp(s_j - max s) V_j / sum_j exp(s_j - max s) with math.fsum
for every sum (page "gfx942 unified attention, from the math up", sections 1
and 2). Only meant for a few hundred scores; used to cross-check the numpy
oracle on tiny cases.
"""
from __future__ import annotations

import math


def brute_row(q, keys, values, scale):
    """q: list of d floats; keys/values: lists of visible rows (lists of d floats)."""
    if not keys:
        return [0.0] * len(q)
    s = [scale * math.fsum(a * b for a, b in zip(q, k)) for k in keys]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    den = math.fsum(w)
    d = len(values[0])
    return [math.fsum(w[j] * values[j][c] for j in range(len(values))) / den for c in range(d)]
