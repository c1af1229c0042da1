"""Materialised fp64 scaled-dot-product attention -- the plain definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows the page "gfx942 unified attention, from the math up":
  * section 1: O = softmax(tau * Q K^T) V with tau = 1/sqrt(d); each output row
    is a convex combination of V rows;
  * section 2: the softmax is evaluated after subtracting the row maximum;
  * section 4: causal masking is aligned to the bottom-right corner, i.e. query
    row i of S_q sees key j iff j <= i + (S_k - S_q);
  * section 5: paged K/V live in a cache [num_blocks, block_size, kv_heads, d];
    sequence row j sits in page block_table[j // block_size] at slot
    j % block_size; a query head h reads KV head floor(h / G), G = heads/kv_heads
    (K/V repeat-interleaved across the group);
  * section 10: gather per sequence, map heads, score, mask, softmax, weight V.

Nothing is tiled or fused: scores for a block of query rows are materialised in
full. Inputs are float64 arrays holding the exact values of the stored
fp16/bf16 inputs. Readings of points the pages leave open:
  * a row with no visible key has output 0 and lse -inf;
  * the per-sequence key length L_b replaces S_k in the mask offset;
  * lse = m + ln(sum_j exp(s_j - m)) in natural log.
"""
from __future__ import annotations

import math

import numpy as np

_ROW_BLOCK = 1024


def kv_head_of(h: int, group: int) -> int:
    """KV head read by query head h: floor(h / G) (repeat_interleave over the group)."""
    return h // group


def is_visible(i, j, L: int, S_q: int, causal: bool):
    """Key j is visible to query row i: j < L, and when causal j <= i + (L - S_q)."""
    vis = j < L
    if causal:
        vis = vis & (j <= i + (L - S_q))
    return vis


def gather_kv(cache: np.ndarray, table_row: np.ndarray, L: int, kvh: int) -> np.ndarray:
    """Rows 0..L-1 of one sequence's keys (or values) for KV head kvh, through its block table."""
    page = cache.shape[1]
    j = np.arange(L)
    return cache[np.asarray(table_row)[j // page], j % page, kvh, :]


def _seq_kv(x: np.ndarray, b: int, kvh: int, L: int, layout: str, block_table) -> np.ndarray:
    if block_table is not None:
        return gather_kv(x, block_table[b], L, kvh)
    if layout == "bshd":
        return x[b, :L, kvh, :]
    return x[b, kvh, :L, :]


def attention_rows(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, rows: np.ndarray, L: int,
                   S_q: int, causal: bool, scale: float, key_range=None, return_weights=False):
    """Attention for a set of query rows of one (sequence, head).

    q_rows: [n, d] queries at positions ``rows`` (0-based among the S_q queries);
    K, V: [L, d] the sequence's keys and values. ``key_range=(lo, hi)`` restricts
    the keys to lo <= j < hi (used for split-KV partials). Returns (O [n, d],
    lse [n]) and, if asked, the weight matrix [n, L].
    """
    rows = np.asarray(rows)
    s = scale * (q_rows @ K.T)
    j = np.arange(K.shape[0])
    vis = is_visible(rows[:, None], j[None, :], L, S_q, causal)
    if key_range is not None:
        lo, hi = key_range
        vis = vis & (j[None, :] >= lo) & (j[None, :] < hi)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.where(vis, np.exp(s - m_safe[:, None]), 0.0)
    denom = w.sum(axis=1)
    empty = denom == 0.0
    a = w / np.where(empty, 1.0, denom)[:, None]
    O = a @ V
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, denom)))
    if return_weights:
        return O, lse, a
    return O, lse


def attention(q, k, v, *, causal: bool, scale=None, layout: str = "bshd", block_table=None,
              seqlens_k=None, q_index=None, key_range=None):
    """Attention forward for a whole batch.

    q: [B, S_q, Hq, d] (bshd) or [B, Hq, S_q, d] (bhsd), float64.
    k, v: paged caches [num_blocks, block_size, Hkv, d] when ``block_table``
    ([B, max_blocks] ints) is given, else dense tensors in ``layout`` with Hkv
    heads and S_k rows. ``seqlens_k`` ([B]) defaults to S_k (dense) or is
    required (paged). ``q_index`` optionally selects which query positions to
    evaluate (all sequences and heads). Returns (O in q's layout restricted to
    q_index, lse [B, Hq, n]).
    """
    if layout not in ("bshd", "bhsd"):
        raise ValueError("layout must be 'bshd' or 'bhsd'")
    qh = q if layout == "bhsd" else q.transpose(0, 2, 1, 3)      # [B, Hq, S_q, d]
    B, Hq, S_q, d = qh.shape
    Hkv = k.shape[2] if (block_table is not None or layout == "bshd") else k.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if seqlens_k is None:
        if block_table is not None:
            raise ValueError("paged K/V needs seqlens_k")
        S_k = k.shape[1] if layout == "bshd" else k.shape[2]
        seqlens_k = [S_k] * B
    rows_all = np.arange(S_q) if q_index is None else np.asarray(q_index)
    n = rows_all.size
    O = np.zeros((B, Hq, n, d), dtype=np.float64)
    lse = np.zeros((B, Hq, n), dtype=np.float64)
    for b in range(B):
        L = int(seqlens_k[b])
        for h in range(Hq):
            kvh = kv_head_of(h, G)
            K = _seq_kv(k, b, kvh, L, layout, block_table)
            V = _seq_kv(v, b, kvh, L, layout, block_table)
            for r0 in range(0, n, _ROW_BLOCK):
                rows = rows_all[r0:r0 + _ROW_BLOCK]
                o, l = attention_rows(qh[b, h, rows, :], K, V, rows, L, S_q, causal, scale,
                                      key_range=key_range)
                O[b, h, r0:r0 + rows.size] = o
                lse[b, h, r0:r0 + rows.size] = l
    if layout == "bshd":
        O = O.transpose(0, 2, 1, 3)
    return O, lse
