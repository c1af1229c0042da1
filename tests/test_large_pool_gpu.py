"""K/V buffers larger than 4 GiB. The pages that a block table names lie past byte
offset 2^32 of the pool and on both sides of 2^31 (and dense K/V put a sequence or heads
past those offsets), so the kernels' copy addresses carry a high word and low words with
bit 31 set, through the wave-uniform base plus per-lane offset copies (prefill) and the
per-lane address copies (decode, ragged tails). Every launch must match the fp64 oracle
run on the same keys stored compactly."""
import dataclasses

import numpy as np
import pytest
import torch

from attn_workloads import DecodeCase, PrefillCase as P, make_decode_inputs, make_prefill_inputs
from gpu_util import (TOL, TORCH_DT, dev, dev_i32, lse_tolerance, max_abs_err, oracle_decode, oracle_prefill,
                      say, to_f64)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

GIB = 1 << 30


def spread_ids(n_used: int, page_bytes: int, seed: int):
    """Pool size (pages) and a page id for each of n_used compact pages: a third just
    below and above byte offset 2^31, a third past 2^32, the rest anywhere in the pool."""
    total = (4 * GIB + 256 * (1 << 20)) // page_bytes
    rng = np.random.default_rng(seed)
    at31 = (2 * GIB) // page_bytes
    at32 = (4 * GIB) // page_bytes
    n1 = n2 = -(-n_used // 3)
    near31 = rng.choice(np.arange(at31 - n_used, at31 + n_used), size=n1, replace=False)
    past32 = rng.choice(np.arange(at32, total), size=n2, replace=False)
    rest = np.setdiff1d(np.arange(total), np.concatenate([near31, past32]))
    ids = rng.permutation(np.concatenate([near31, past32, rng.choice(rest, size=n_used, replace=False)])[:n_used])
    assert len(np.unique(ids)) == n_used and ids.max() < total
    assert (ids >= at32).any() and ((ids >= at31) & (ids < at32)).any() and (ids < at31).any()
    return total, ids.astype(np.int64)


def big_pool(pages: np.ndarray, dtype: str, total: int, ids: np.ndarray) -> torch.Tensor:
    """A [total, 64, Hkv, d] device pool holding compact page i at page ids[i]; the
    other pages are never named by the table and stay unwritten."""
    pool = torch.empty((total,) + pages.shape[1:], dtype=TORCH_DT[dtype], device="cuda")
    pool[torch.from_numpy(ids).cuda()] = dev(pages, dtype)
    return pool


PREFILL = [
    # (case, kv_splits): the one-group four-wave form, its tail split, the two-group
    # causal form, the narrow d = 256 kernel and its split, d = 64, the paired two-group
    # form (512 query blocks), the eight-wave form (1024 workgroups)
    (P("bf16_d128_gqa4_noncausal_big_pool", 2, 8, 2, 300, 900, 128, "bf16", False, "paged",
       seqlens_k=(900, 640)), (0, 4)),
    (P("f16_d128_gqa4_causal_big_pool", 2, 8, 2, 500, 1200, 128, "f16", True, "paged",
       seqlens_k=(1200, 700)), (0,)),
    (P("bf16_d256_gqa2_causal_big_pool", 2, 4, 2, 300, 700, 256, "bf16", True, "paged",
       seqlens_k=(700, 500)), (0, 3)),
    (P("bf16_d64_mha_noncausal_big_pool", 2, 4, 4, 200, 1000, 64, "bf16", False, "paged",
       seqlens_k=(1000, 333)), (0,)),
    (P("f16_d128_gqa4_causal_paired_big_pool", 1, 32, 8, 2048, 2048, 128, "f16", True, "paged"), (0,)),
    (P("bf16_d128_gqa4_noncausal_wg8_big_pool", 4, 32, 8, 2048, 700, 128, "bf16", False, "paged",
       seqlens_k=(700, 640, 65, 700)), (0,)),
]


@pytest.mark.parametrize("case,splits", PREFILL, ids=lambda x: getattr(x, "name", str(x)))
def test_prefill_pages_past_4gib(case, splits):
    from attention_forward_tiled_amd import attn_prefill_fwd
    inp = make_prefill_inputs(case, seed=31)
    nb, page_bytes = inp.k.shape[0], inp.k[0].nbytes
    total, ids = spread_ids(nb, page_bytes, seed=32)
    say(f"prefill, pool of {total} pages ({total * page_bytes / GIB:.2f} GiB each for K and V) {case}")
    k, v = big_pool(inp.k, case.dtype, total, ids), big_pool(inp.v, case.dtype, total, ids)
    table = dev_i32(ids[inp.block_table])
    rows = np.arange(case.seqlen_q)
    if case.seqlen_q > 600:   # every workgroup boundary of the first blocks, the last row, a sample
        rows = np.unique(np.concatenate([[0, 31, 32, 63, 64, 127, 128, 255, 256, case.seqlen_q - 1],
                                         np.random.default_rng(3).choice(case.seqlen_q, 16, replace=False)]))
    Oref, lref = oracle_prefill(inp, q_index=rows)
    q, sl = dev(inp.q, case.dtype), dev_i32(inp.seqlens_k)
    for s in splits:
        say(f"  kv_splits={s}")
        out = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
        lse = torch.full((case.batch, case.heads_q, case.seqlen_q), float("nan"), device="cuda")
        attn_prefill_fwd(q, k, v, causal=case.causal, block_table=table, seqlens_k=sl,
                         seqlen_k=case.seqlen_k, out=out, lse=lse, kv_splits=s)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out).all())
        err = max_abs_err(to_f64(out)[:, rows], Oref)
        say(f"  max abs err {err:.3e} over {rows.size} rows x all (b, h)")
        assert err <= TOL[case.dtype]
        lg = to_f64(lse)[:, :, rows]
        fin = np.isfinite(lref)
        assert (np.isneginf(lg) == np.isneginf(lref)).all()
        assert np.abs(lg[fin] - lref[fin]).max(initial=0.0) <= lse_tolerance(case.dtype)
    del k, v
    torch.cuda.empty_cache()


DECODE = [
    DecodeCase("bf16_g4_d128_big_pool", 4, 8, 2, 128, "bf16", lengths_fixed=(1000, 64, 3000, 1)),
    DecodeCase("f16_g2_d256_big_pool", 3, 4, 2, 256, "f16", lengths_fixed=(700, 129, 1500)),
    DecodeCase("bf16_g8_d64_big_pool", 2, 16, 2, 64, "bf16", lengths_fixed=(2000, 333)),
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: c.name)
def test_decode_pages_past_4gib(case):
    from attention_forward_tiled_amd import attn_decode_fwd
    inp = make_decode_inputs(case, seed=33)
    used = sorted({int(x) for b in range(case.batch)
                   for x in inp.block_table[b, :-(-int(inp.seqlens_k[b]) // 64)]})
    compact = {pg: i for i, pg in enumerate(used)}
    pages_k, pages_v = inp.k_cache[used], inp.v_cache[used]
    total, ids = spread_ids(len(used), pages_k[0].nbytes, seed=34)
    say(f"decode, pool of {total} pages {case}")
    k, v = big_pool(pages_k, case.dtype, total, ids), big_pool(pages_v, case.dtype, total, ids)
    table = np.zeros_like(inp.block_table)
    for b in range(case.batch):
        n = -(-int(inp.seqlens_k[b]) // 64)
        table[b, :n] = [ids[compact[int(x)]] for x in inp.block_table[b, :n]]
    Oref, lref = oracle_decode(inp)
    for s in (1, 16):
        say(f"  num_splits={s}")
        out = torch.full((case.batch, case.heads_q, case.head_dim), float("nan"),
                         dtype=TORCH_DT[case.dtype], device="cuda")
        lse = torch.full((case.batch, case.heads_q), float("nan"), device="cuda")
        attn_decode_fwd(dev(inp.q, case.dtype), k, v, dev_i32(table), dev_i32(inp.seqlens_k),
                        max_seqlen_k=inp.max_seqlen_k, num_splits=s, out=out, lse=lse)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out).all())
        err = max_abs_err(to_f64(out), Oref)
        say(f"  max abs err {err:.3e}")
        assert err <= TOL[case.dtype]
        assert np.abs(to_f64(lse) - lref).max() <= lse_tolerance(case.dtype)
    del k, v
    torch.cuda.empty_cache()


DENSE = [
    # dense K/V of 2^20 keys per sequence (4 GiB per sequence and tensor): the second
    # sequence starts past byte 2^32 (BSHD), or heads 8 and on start past 2^31 (BHSD);
    # only the first keys of each sequence are used
    (P("bf16_d128_gqa2_noncausal_dense_bshd_big", 2, 32, 16, 300, 1 << 20, 128, "bf16", False, "dense",
       seqlens_k=(500, 700)), 700),
    (P("f16_d128_gqa2_causal_dense_bhsd_big", 2, 32, 16, 300, 1 << 20, 128, "f16", True, "dense",
       layout="bhsd", seqlens_k=(640, 333)), 640),
]


@pytest.mark.parametrize("case,used", DENSE, ids=lambda x: getattr(x, "name", str(x)))
def test_prefill_dense_kv_past_4gib(case, used):
    from attention_forward_tiled_amd import attn_prefill_fwd
    small = dataclasses.replace(case, seqlen_k=used)
    inp = make_prefill_inputs(small, seed=35)
    bhsd = case.layout == "bhsd"
    shape = (case.batch, case.heads_kv, case.seqlen_k, case.head_dim) if bhsd else \
        (case.batch, case.seqlen_k, case.heads_kv, case.head_dim)
    say(f"prefill, dense K/V of {2 * np.prod(shape) / GIB:.1f} GiB each {case}")
    k = torch.empty(shape, dtype=TORCH_DT[case.dtype], device="cuda")
    v = torch.empty(shape, dtype=TORCH_DT[case.dtype], device="cuda")
    if bhsd:
        k[:, :, :used], v[:, :, :used] = dev(inp.k, case.dtype), dev(inp.v, case.dtype)
    else:
        k[:, :used], v[:, :used] = dev(inp.k, case.dtype), dev(inp.v, case.dtype)
    Oref, lref = oracle_prefill(inp)
    q = dev(inp.q, case.dtype)
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full((case.batch, case.heads_q, case.seqlen_q), float("nan"), device="cuda")
    attn_prefill_fwd(q, k, v, causal=case.causal, seqlens_k=dev_i32(inp.seqlens_k), seqlen_k=case.seqlen_k,
                     layout=case.layout, out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    err = max_abs_err(to_f64(out), Oref)
    say(f"  max abs err {err:.3e}")
    assert err <= TOL[case.dtype]
    assert np.abs(to_f64(lse) - lref).max() <= lse_tolerance(case.dtype)
    del k, v
    torch.cuda.empty_cache()
