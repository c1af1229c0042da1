"""Helpers shared by the GPU parity tests: device copies of the seeded inputs,
calls through the C ABI (via the binding), and oracle evaluations."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from attn_workloads import bits_to_f64

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
TOL = {"f16": 2e-2, "bf16": 4e-2}
TOL_PRECISE = 1e-4
# unit roundoff of the 16-bit type that P is rounded to before the P.V product
UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def lse_tolerance(dtype: str, precise: bool = False) -> float:
    """One lse tolerance for prefill and decode. Both paths sum the row denominator l
    from P as it enters the P.V product: rounded to nearest even in the input type, or
    (precise mode) as the hi + lo pair that carries P at about fp32 precision. Where one
    key dominates a row, the rounding of its term (relative <= u) reaches ln l
    unaveraged, so lse may be off by up to u; 1e-4 covers fp32 rounding."""
    return 1e-4 if precise else UNIT_ROUNDOFF[dtype] + 1e-4


def say(msg: str):
    """Name the case before any GPU work, flushed, so a failing run says where it was."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev(bits: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TORCH_DT[dtype])
    return t.cuda()


def dev_i32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def tolerance(case) -> float:
    return TOL_PRECISE if getattr(case, "precise", False) else TOL[case.dtype]


def gpu_prefill(inp, *, with_lse=False, out_dtype=None, out_round="rtne", kv_splits=0):
    """Run attn_prefill_fwd on the seeded inputs; returns (O, lse) as float64 numpy.

    The output (and lse) buffers are filled with NaN before the launch and the whole
    output must come back finite, so a row the kernels never write fails even where a
    test compares only sampled rows with the oracle."""
    from attention_forward_tiled_amd import attn_prefill_fwd
    c = inp.case
    q, k, v = dev(inp.q, c.dtype), dev(inp.k, c.dtype), dev(inp.v, c.dtype)
    bt = dev_i32(inp.block_table) if inp.block_table is not None else None
    sl = dev_i32(inp.seqlens_k) if (inp.block_table is not None or c.seqlens_k is not None) else None
    odt = TORCH_DT[out_dtype or c.o_dtype]
    lse = None
    if with_lse:
        lse = torch.full((c.batch, c.heads_q, c.seqlen_q), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full(q.shape, float("nan"), dtype=odt, device="cuda")
    o = attn_prefill_fwd(q, k, v, causal=c.causal, block_table=bt, seqlens_k=sl,
                         seqlen_k=c.seqlen_k, layout=c.layout, out=out, lse=lse,
                         precise=c.precise, out_round=out_round, kv_splits=kv_splits)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()), "output rows left unwritten (NaN) or non-finite"
    if lse is not None:
        assert not bool(torch.isnan(lse).any()), "lse entries left unwritten"
    return to_f64(o), (to_f64(lse) if lse is not None else None)


def oracle_prefill(inp, q_index=None):
    c = inp.case
    q = bits_to_f64(inp.q, c.dtype)
    k = bits_to_f64(inp.k, c.dtype)
    v = bits_to_f64(inp.v, c.dtype)
    return oracle.attention(q, k, v, causal=c.causal, layout=c.layout, block_table=inp.block_table,
                            seqlens_k=inp.seqlens_k, q_index=q_index)


def oracle_decode(inp, seqs=None, per_call=4):
    """fp64 oracle on the chosen sequences (default: all), ``per_call`` sequences at a
    time: their pages are copied out of the pool and upcast, so host memory stays
    bounded by the longest few sequences, not the whole cache. Returns (O [n, Hq, d],
    lse [n, Hq])."""
    c = inp.case
    seqs = list(range(c.batch)) if seqs is None else list(seqs)
    O_all, lse_all = [], []
    for i0 in range(0, len(seqs), per_call):
        part = seqs[i0:i0 + per_call]
        tables, pages = [], []
        for b in part:
            n = -(-int(inp.seqlens_k[b]) // 64)
            tables.append(list(range(len(pages), len(pages) + n)))
            pages.extend(int(x) for x in inp.block_table[b, :n])
        width = max(1, max(len(t) for t in tables))
        table = np.zeros((len(part), width), dtype=np.int64)
        for i, t in enumerate(tables):
            table[i, :len(t)] = t
        pages = pages or [0]
        k = bits_to_f64(inp.k_cache[pages], c.dtype)
        v = bits_to_f64(inp.v_cache[pages], c.dtype)
        q = bits_to_f64(inp.q[part], c.dtype)                      # [n, 1, Hq, d]
        O, lse = oracle.attention(q, k, v, causal=False, block_table=table,
                                  seqlens_k=inp.seqlens_k[part])
        del k, v
        O_all.append(O[:, 0])
        lse_all.append(lse[:, :, 0])
    return np.concatenate(O_all), np.concatenate(lse_all)


def max_abs_err(a: np.ndarray, b: np.ndarray) -> float:
    if a.shape != b.shape:
        raise AssertionError(f"shape mismatch {a.shape} vs {b.shape}")
    if not np.isfinite(a).all():
        return float("inf")
    return float(np.abs(a - b).max()) if a.size else 0.0


def check_bf16_rounding(o_bf16: np.ndarray, o_f32: np.ndarray, mode: str):
    """Relations that the bf16 output of a launch must satisfy against the fp32 output
    of the same launch (same arithmetic, only the final conversion differs): it lies
    on the bf16 grid, within half a bf16 unit for the nearest modes and below it in
    magnitude for RTZ; at exact ties it rounds to the even neighbour (RTNE) or away
    from zero (RTNA)."""
    x = o_f32.astype(np.float32)
    r = o_bf16.astype(np.float32)
    assert ((r.view(np.uint32) & 0xFFFF) == 0).all(), "output not on the bf16 grid"
    xb = x.view(np.uint32)
    nz = (xb & 0x7FFFFFFF) >= 0x00800000                      # normal fp32 values
    ulp = np.exp2(np.floor(np.log2(np.abs(x[nz].astype(np.float64)))) - 7)
    diff = np.abs(r[nz].astype(np.float64) - x[nz].astype(np.float64))
    if mode == "rtz":
        assert (np.abs(r[nz]) <= np.abs(x[nz])).all() and (diff < ulp).all()
    else:
        assert (diff <= ulp / 2).all()
        tie = nz & ((xb & 0xFFFF) == 0x8000)
        if tie.any():
            if mode == "rtna":
                assert (np.abs(r[tie]) > np.abs(x[tie])).all()
            else:
                assert ((r[tie].view(np.uint32) >> 16) & 1 == 0).all()
    return int((nz & ((xb & 0xFFFF) == 0x8000)).sum())
