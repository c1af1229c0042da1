"""Seeded input generation (numpy, host memory).

Values are float32 N(0,1) draws, multiplied by the case's exact power-of-two
``value_scale`` and rounded (round-to-nearest-even) to the storage dtype. Arrays
hold the raw 16-bit storage patterns (``uint16``); ``bits_to_f64`` upcasts them
exactly.

Streams: every array has a stream id (Q = 1, K = 2, V = 3); its elements, in
C order, are cut into chunks of 2^22 and chunk i is drawn from
``Generator(PCG64(SeedSequence([seed, stream, i])))``, so large arrays fill in
parallel threads yet depend only on the seed. Integer structure (decode key
lengths, then the page permutation) comes from ``PCG64(SeedSequence([seed, 0]))``.
Prefill Q/K/V are drawn in logical BSHD order whatever the storage. Storage
slots past a sequence's last key are filled with NaN when ``poison`` is set,
so a kernel that lets them reach the output fails parity.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import PAGE, DecodeCase, PrefillCase

NAN_BITS = {"f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}
_CHUNK = 1 << 22


def round_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to fp16/bf16 (nearest, ties to even); return the bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32)
        nan = np.isnan(x)
        r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
        if nan.any():
            r[nan] = NAN_BITS["bf16"]
        return r
    raise ValueError(f"unknown storage dtype {dtype!r}")


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of stored fp16/bf16 patterns to float64."""
    return bits_to_f32(bits, dtype).astype(np.float64)


def _bf16_bits_inplace(x: np.ndarray) -> np.ndarray:
    """RTNE float32 -> bf16 for finite values, reusing x's buffer."""
    u = x.view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def _normal_bits(seed: int, stream: int, shape, dtype: str, scale: float) -> np.ndarray:
    """Draw N(0,1)*scale in float32 chunk by chunk (threads) and round to the storage dtype."""
    out = np.empty(int(np.prod(shape)), dtype=np.uint16)
    n = out.size

    def fill(i):
        s, e = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, i])))
        x = rng.standard_normal(e - s, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[s:e] = _bf16_bits_inplace(x) if dtype == "bf16" else round_to_bits(x, dtype)

    n_chunks = -(-n // _CHUNK)
    if n_chunks <= 1:
        for i in range(n_chunks):
            fill(i)
    else:
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1, n_chunks)) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out.reshape(shape)


@dataclass
class PrefillInputs:
    case: PrefillCase
    q: np.ndarray                   # uint16, [B,S_q,Hq,d] (bshd) or [B,Hq,S_q,d] (bhsd)
    k: np.ndarray                   # paged: [num_blocks,64,Hkv,d]; dense: like q with Hkv, S_k
    v: np.ndarray
    block_table: Optional[np.ndarray]  # int32 [B, max_blocks] (paged) or None (dense)
    seqlens_k: np.ndarray           # int32 [B]


@dataclass
class DecodeInputs:
    case: DecodeCase
    q: np.ndarray                   # uint16, [B,1,Hq,d] (bshd) or [B,Hq,1,d] (bhsd)
    k_cache: np.ndarray             # uint16, [num_blocks,64,Hkv,d]
    v_cache: np.ndarray
    block_table: np.ndarray         # int32 [B, max_blocks]; unused entries are 0
    seqlens_k: np.ndarray           # int32 [B]

    @property
    def max_seqlen_k(self) -> int:
        return int(self.seqlens_k.max()) if self.seqlens_k.size else 0


def make_prefill_inputs(case: PrefillCase, seed: int = 0) -> PrefillInputs:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0])))
    B, Sq, Sk, Hq, Hkv, d = case.batch, case.seqlen_q, case.seqlen_k, case.heads_q, case.heads_kv, case.head_dim
    lens = np.asarray(case.lengths(), dtype=np.int32)
    if lens.shape != (B,) or (lens < 0).any() or (lens > Sk).any():
        raise ValueError("seqlens_k must have one entry per sequence, each in [0, seqlen_k]")
    q = _normal_bits(seed, 1, (B, Sq, Hq, d), case.dtype, case.value_scale)
    k = _normal_bits(seed, 2, (B, Sk, Hkv, d), case.dtype, case.value_scale)
    v = _normal_bits(seed, 3, (B, Sk, Hkv, d), case.dtype, case.value_scale)
    if case.poison:
        nan = NAN_BITS[case.dtype]
        for b in range(B):
            k[b, lens[b]:] = nan
            v[b, lens[b]:] = nan
    if case.layout == "bhsd":
        q = np.ascontiguousarray(q.transpose(0, 2, 1, 3))
    elif case.layout != "bshd":
        raise ValueError(f"unknown layout {case.layout!r}")

    if case.kv == "dense":
        if case.layout == "bhsd":
            k = np.ascontiguousarray(k.transpose(0, 2, 1, 3))
            v = np.ascontiguousarray(v.transpose(0, 2, 1, 3))
        return PrefillInputs(case, q, k, v, None, lens)

    if case.kv != "paged":
        raise ValueError(f"unknown kv storage {case.kv!r}")
    pages_per_seq = -(-Sk // PAGE)
    num_blocks = B * pages_per_seq
    if case.table == "identity":
        perm = np.arange(num_blocks, dtype=np.int64)
    elif case.table == "random":
        perm = rng.permutation(num_blocks)
    else:
        raise ValueError(f"unknown table kind {case.table!r}")
    table = perm.reshape(B, pages_per_seq).astype(np.int32)
    fill = NAN_BITS[case.dtype] if case.poison else np.uint16(0)
    kc = np.full((num_blocks, PAGE, Hkv, d), fill, dtype=np.uint16)
    vc = np.full((num_blocks, PAGE, Hkv, d), fill, dtype=np.uint16)
    for b in range(B):
        for j in range(pages_per_seq):
            lo, hi = j * PAGE, min(Sk, (j + 1) * PAGE)
            kc[table[b, j], : hi - lo] = k[b, lo:hi]
            vc[table[b, j], : hi - lo] = v[b, lo:hi]
    return PrefillInputs(case, q, kc, vc, table, lens)


def make_decode_inputs(case: DecodeCase, seed: int = 0) -> DecodeInputs:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0])))
    B, Hq, Hkv, d = case.batch, case.heads_q, case.heads_kv, case.head_dim
    if case.lengths_fixed is not None:
        lens = np.asarray(case.lengths_fixed, dtype=np.int32)
        if lens.shape != (B,):
            raise ValueError("lengths_fixed must have one entry per sequence")
    else:
        lens = rng.integers(case.len_lo, case.len_hi, size=B, endpoint=True).astype(np.int32)
    q = _normal_bits(seed, 1, (B, 1, Hq, d), case.dtype, 1.0)
    if case.layout == "bhsd":
        q = np.ascontiguousarray(q.transpose(0, 2, 1, 3))
    elif case.layout != "bshd":
        raise ValueError(f"unknown layout {case.layout!r}")
    pages = [-(-int(L) // PAGE) for L in lens]
    num_blocks = max(1, sum(pages))
    kc = _normal_bits(seed, 2, (num_blocks, PAGE, Hkv, d), case.dtype, 1.0)
    vc = _normal_bits(seed, 3, (num_blocks, PAGE, Hkv, d), case.dtype, 1.0)
    perm = rng.permutation(num_blocks).astype(np.int32)
    max_blocks = max(1, max(pages) if pages else 1)
    table = np.zeros((B, max_blocks), dtype=np.int32)
    start = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[start:start + n]
        start += n
    if case.poison:
        nan = NAN_BITS[case.dtype]
        for b, L in enumerate(lens):
            tail = int(L) % PAGE
            if tail:
                last = table[b, pages[b] - 1]
                kc[last, tail:] = nan
                vc[last, tail:] = nan
        used = set(int(x) for x in perm[:start])
        for blk in range(num_blocks):
            if blk not in used:
                kc[blk] = nan
                vc[blk] = nan
    return DecodeInputs(case, q, kc, vc, table, lens)
