"""Workload descriptions: shapes, dtypes and structure of the synthetic inputs.

The five named workloads follow the shapes the attention pages measure
(page "gfx942 unified attention -- parity + benchmark harness", sections
"The shape set" and "How the harness maps a dense SDPA problem onto the paged
kernel"; page 7minutos.es / MoonMath, section "Punto de referencia" for the
(4, 16, 16384) bf16 d=128 shape). Values are N(0,1) draws rounded (RTNE) to the
storage dtype; paged K/V live in 64-token pages reached through a block table.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple

PAGE = 64  # tokens per KV page (block_size), equal to the KV tile width T


@dataclass(frozen=True)
class PrefillCase:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen_q: int
    seqlen_k: int
    head_dim: int
    dtype: str = "f16"            # storage dtype of Q/K/V: "f16" | "bf16"
    causal: bool = True           # bottom-right aligned causal mask
    kv: str = "paged"             # "paged" (64-token pages + block table) | "dense"
    table: str = "random"         # paged only: "identity" | "random" page order
    layout: str = "bshd"          # Q/O layout (and dense K/V): "bshd" | "bhsd"
    value_scale: float = 1.0      # N(0,1) draws are multiplied by this (exact power of two)
    out_dtype: Optional[str] = None   # None -> same as dtype; "f32" allowed
    precise: bool = False         # keep P at ~fp32 precision in P.V (hi+lo split)
    seqlens_k: Optional[Tuple[int, ...]] = None  # per-sequence key lengths (<= seqlen_k)
    poison: bool = True           # fill storage slots past a sequence's keys with NaN

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv

    @property
    def o_dtype(self) -> str:
        return self.out_dtype or self.dtype

    def lengths(self) -> Tuple[int, ...]:
        return self.seqlens_k if self.seqlens_k is not None else (self.seqlen_k,) * self.batch

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs a query head sees, summed over the batch."""
        total = 0
        for L in self.lengths():
            if not self.causal:
                total += self.seqlen_q * L
            else:
                off = L - self.seqlen_q
                for i in range(self.seqlen_q):
                    total += max(0, min(L, i + off + 1))
        return total

    def flops_exact(self) -> int:
        """2 flops per MAC for each of Q.K^T and P.V over the visible pairs."""
        return 4 * self.head_dim * self.heads_q * self.visible_pairs()

    def flops_half_convention(self) -> int:
        """Dense 4*d*S_q*S_k per head, halved when causal ("causal counted as half")."""
        dense = 4 * self.head_dim * self.heads_q * self.seqlen_q * sum(self.lengths())
        return dense // 2 if self.causal else dense

    def with_(self, **kw) -> "PrefillCase":
        return replace(self, **kw)


@dataclass(frozen=True)
class DecodeCase:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    dtype: str = "bf16"
    len_lo: int = 1024            # key lengths drawn uniformly from [len_lo, len_hi]
    len_hi: int = 65536
    num_splits: int = 16
    layout: str = "bshd"
    lengths_fixed: Optional[Tuple[int, ...]] = None  # overrides the draw when given
    poison: bool = True

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv

    def with_(self, **kw) -> "DecodeCase":
        return replace(self, **kw)


CONFIGS = {
    # Oracle bring-up: one head, 128 tokens, contiguous pages, P and O kept at fp32.
    "tiny_causal_f16_d64": PrefillCase(
        "tiny_causal_f16_d64", batch=1, heads_q=1, heads_kv=1, seqlen_q=128, seqlen_k=128,
        head_dim=64, dtype="f16", causal=True, kv="paged", table="identity",
        out_dtype="f32", precise=True),
    # Causal GQA prefill over a randomly ordered page pool.
    "gqa_causal_paged_f16_s2048": PrefillCase(
        "gqa_causal_paged_f16_s2048", batch=1, heads_q=32, heads_kv=8, seqlen_q=2048,
        seqlen_k=2048, head_dim=128, dtype="f16", causal=True, kv="paged", table="random"),
    # Chunked prefill: 512 new queries appended to 4096 keys, bottom-right causal.
    "chunked_prefill_bf16_512x4096": PrefillCase(
        "chunked_prefill_bf16_512x4096", batch=4, heads_q=16, heads_kv=4, seqlen_q=512,
        seqlen_k=4096, head_dim=128, dtype="bf16", causal=True, kv="paged", table="random"),
    # Long-KV split decode over a random page pool, key lengths U[1024, 65536].
    "splitkv_decode_bf16_64k": DecodeCase(
        "splitkv_decode_bf16_64k", batch=32, heads_q=32, heads_kv=8, head_dim=128,
        dtype="bf16", len_lo=1024, len_hi=65536, num_splits=16),
    # Head sizes 256 and 64 (the other two tiled paths): causal MHA self-attention over
    # dense BSHD K/V, 4096 positions.
    "causal_mha_bf16_d256_s4096": PrefillCase(
        "causal_mha_bf16_d256_s4096", batch=2, heads_q=16, heads_kv=16, seqlen_q=4096,
        seqlen_k=4096, head_dim=256, dtype="bf16", causal=True, kv="dense", layout="bshd",
        poison=False),
    "causal_mha_f16_d64_s4096": PrefillCase(
        "causal_mha_f16_d64_s4096", batch=8, heads_q=32, heads_kv=32, seqlen_q=4096,
        seqlen_k=4096, head_dim=64, dtype="f16", causal=True, kv="dense", layout="bshd",
        poison=False),
    # Long non-causal MHA self-attention, dense BSHD K/V, inputs 0.5*N(0,1).
    # Chunked prefill of two short chunks: 2 x 4 KV heads x 8 query blocks = 64 items,
    # too few for the CUs (the causal few-item split).
    "chunked_small_bf16_2x256x4096": PrefillCase(
        "chunked_small_bf16_2x256x4096", batch=2, heads_q=16, heads_kv=4, seqlen_q=256,
        seqlen_k=4096, head_dim=128, dtype="bf16", causal=True, kv="paged", table="random"),
    # A launch whose last round of work items is a quarter full (25 heads x 64 query
    # blocks of 256 rows on 256 CUs): the shape of the prefill tail split.
    "tail_noncausal_bf16_h25_s16384": PrefillCase(
        "tail_noncausal_bf16_h25_s16384", batch=1, heads_q=25, heads_kv=25, seqlen_q=16384,
        seqlen_k=16384, head_dim=128, dtype="bf16", causal=False, kv="dense",
        layout="bshd", value_scale=0.5, poison=False),
    "long_noncausal_bf16_s16384": PrefillCase(
        "long_noncausal_bf16_s16384", batch=4, heads_q=16, heads_kv=16, seqlen_q=16384,
        seqlen_k=16384, head_dim=128, dtype="bf16", causal=False, kv="dense",
        layout="bshd", value_scale=0.5, poison=False),
}


def config(name: str):
    return CONFIGS[name]
