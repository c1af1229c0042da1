"""Split-KV partials and their log-sum-exp merge, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The page "gfx942 unified attention, from the math up", section 8, splits the
key dimension of a decode query across workgroups and combines the partial
softmax-weighted outputs. Reading used here: a split s over keys [lo, hi)
yields its own normalised output O_s = softmax(s restricted to the split) V and
lse_s = m_s + ln(sum over the split of exp(s_j - m_s)); an empty split has
lse_s = -inf and O_s = 0. The merge is
    M = max_s lse_s,  w_s = exp(lse_s - M),  O = sum_s w_s O_s / sum_s w_s,
which equals the unsplit softmax output because exp(lse_s) is the split's
share of the full softmax denominator.
"""
from __future__ import annotations

import numpy as np

from .materialised import attention


def lse_combine(partial_o: np.ndarray, partial_lse: np.ndarray):
    """Merge partials [..., S, d] / [..., S] into (O [..., d], lse [...])."""
    po = np.asarray(partial_o, dtype=np.float64)
    pl = np.asarray(partial_lse, dtype=np.float64)
    M = pl.max(axis=-1)
    finite = np.isfinite(M)
    M_safe = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(pl), np.exp(pl - M_safe[..., None]), 0.0)
    den = w.sum(axis=-1)
    O = np.einsum("...s,...sd->...d", w, np.where(np.isfinite(pl)[..., None], po, 0.0))
    O = np.where(finite[..., None], O / np.where(finite, den, 1.0)[..., None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(finite, M_safe + np.log(np.where(finite, den, 1.0)), -np.inf)
    return O, lse


def split_partials(q, k, v, *, bounds, causal=False, scale=None, layout="bshd",
                   block_table=None, seqlens_k=None):
    """Per-split (O_s, lse_s) for key ranges ``bounds`` = [(lo, hi), ...].

    Returns partial_o [B, Hq, S_q, S, d] and partial_lse [B, Hq, S_q, S] (query
    axis kept so prefill splits work too).
    """
    outs, lses = [], []
    for lo, hi in bounds:
        O, lse = attention(q, k, v, causal=causal, scale=scale, layout=layout,
                           block_table=block_table, seqlens_k=seqlens_k, key_range=(lo, hi))
        Oh = O if layout == "bhsd" else O.transpose(0, 2, 1, 3)   # [B, Hq, S_q, d]
        outs.append(Oh)
        lses.append(lse)
    return np.stack(outs, axis=3), np.stack(lses, axis=3)
