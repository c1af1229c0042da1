"""Brute-force online (streaming) softmax -- a checker for ``oracle.materialised``.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Evaluates one query row at a time by walking the keys in tiles of an arbitrary
width T and carrying the three running quantities of the page "gfx942 unified
attention, from the math up", section 3: the running maximum m (start -inf),
the running denominator l (start 0) and the un-normalised output o (start 0).
Per tile: m_new = max(m, max of the tile's scores); alpha = exp(m - m_new);
p_j = exp(s_j - m_new); l = alpha*l + sum p; o = alpha*o + sum p_j V_j.
After the last tile O = o / l.

It deliberately re-implements its own page gather, head map and mask instead of
importing them from ``oracle.materialised``, so that it checks that module rather
than repeating it.
"""
from __future__ import annotations

import math

import numpy as np


def _row_keys(cache_or_dense, b, kvh, L, block_table, layout):
    if block_table is not None:
        page = cache_or_dense.shape[1]
        out = np.empty((L, cache_or_dense.shape[3]), dtype=np.float64)
        for j in range(L):
            out[j] = cache_or_dense[block_table[b][j // page], j % page, kvh]
        return out
    if layout == "bshd":
        return np.array(cache_or_dense[b, :L, kvh], dtype=np.float64)
    return np.array(cache_or_dense[b, kvh, :L], dtype=np.float64)


def online_row(q, K, V, i, L, S_q, causal, scale, tile):
    """One query row (position i) against keys K[:L], V[:L], tiles of width ``tile``."""
    d = V.shape[1]
    m = -math.inf
    ell = 0.0
    o = np.zeros(d, dtype=np.float64)
    limit = L
    if causal:
        limit = min(L, i + (L - S_q) + 1)   # keys beyond this are in the row's future
    for t0 in range(0, L, tile):
        t1 = min(L, t0 + tile)
        s = np.array([scale * float(np.dot(q, K[j])) if j < limit else -math.inf
                      for j in range(t0, t1)])
        tile_max = s.max()
        m_new = max(m, tile_max)
        if m_new == -math.inf:          # nothing visible yet: state stays at its start
            continue
        alpha = math.exp(m - m_new)     # exp(-inf) = 0 on the first visible tile
        p = np.array([math.exp(x - m_new) if x != -math.inf else 0.0 for x in s])
        ell = alpha * ell + p.sum()
        o = alpha * o
        for jj, pj in enumerate(p):
            if pj != 0.0:
                o = o + pj * V[t0 + jj]
        m = m_new
    if ell == 0.0:
        return np.zeros(d), -math.inf
    return o / ell, m + math.log(ell)


def online_attention_rows(q, k, v, *, b, h, rows, causal, tile, scale=None, layout="bshd",
                          block_table=None, seqlens_k=None):
    """Online-softmax output for query rows ``rows`` of sequence b, query head h.

    Same argument conventions as ``oracle.attention.attention``. Returns
    (O [len(rows), d], lse [len(rows)]).
    """
    qh = q if layout == "bhsd" else np.transpose(q, (0, 2, 1, 3))
    Hq, S_q, d = qh.shape[1], qh.shape[2], qh.shape[3]
    if block_table is not None or layout == "bshd":
        Hkv = k.shape[2]
    else:
        Hkv = k.shape[1]
    group = Hq // Hkv
    kvh = h // group
    if seqlens_k is not None:
        L = int(seqlens_k[b])
    else:
        L = k.shape[1] if layout == "bshd" else k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    K = _row_keys(k, b, kvh, L, block_table, layout)
    V = _row_keys(v, b, kvh, L, block_table, layout)
    outs, lses = [], []
    for i in rows:
        o, l = online_row(np.asarray(qh[b, h, i], dtype=np.float64), K, V, int(i), L, S_q,
                          causal, scale, tile)
        outs.append(o)
        lses.append(l)
    return np.array(outs), np.array(lses)
