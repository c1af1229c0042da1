"""HIP-graph capture of the entry points (torch.cuda.CUDAGraph) and replay.

With out, lse and the decode workspace passed in, a call launches kernels only: no
allocation, no memset node, no host synchronisation, so it can be captured once and
replayed. Key lengths, packed-query offsets and query values are read on the device,
so they may change in place between replays. Every replay is checked bit for bit
against an eager call on the same inputs (the same kernels in the same order), with
the program's own eager work and synchronisations in between, and the replays on the
original and on shortened lengths against the fp64 oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from attn_workloads import DecodeCase, PrefillCase, bits_to_f64, make_decode_inputs, make_prefill_inputs
from gpu_util import TOL, dev, dev_i32, max_abs_err, oracle_decode, say, to_f64, tolerance

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

REPLAYS = 4


def shorter_lengths(lens, rng):
    """New key lengths, each at most the original (pages past it stay mapped), some 0."""
    new = np.array([rng.integers(0, int(L) + 1) for L in lens], dtype=np.int32)
    new[rng.integers(0, len(new))] = 0
    return new


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                       b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))


@pytest.mark.parametrize("splits", [1, 16])
def test_decode_graph_replays(splits):
    from attention_forward_tiled_amd import attn_decode_fwd, attn_decode_workspace_bytes
    case = DecodeCase("graph_bf16_g4_d128", 4, 16, 4, 128, "bf16", lengths_fixed=(3000, 65, 1, 8191))
    say(f"decode graph capture, splits={splits}, {case}")
    inp = make_decode_inputs(case, seed=21)
    B, Hq, d = case.batch, case.heads_q, case.head_dim
    q = dev(inp.q, case.dtype)
    kc, vc = dev(inp.k_cache, case.dtype), dev(inp.v_cache, case.dtype)
    bt, sl = dev_i32(inp.block_table), dev_i32(inp.seqlens_k)
    ws = torch.empty(attn_decode_workspace_bytes(B, Hq, splits, d), dtype=torch.uint8, device="cuda")
    ws_eager = torch.empty_like(ws)

    def run(o, lse, w):
        attn_decode_fwd(q, kc, vc, bt, sl, max_seqlen_k=inp.max_seqlen_k, num_splits=splits,
                        out=o, lse=lse, workspace=w)

    out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    run(out, lse, ws)                                  # eager warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(out, lse, ws)
    torch.cuda.synchronize()

    rng = np.random.default_rng(7)
    lens = inp.seqlens_k
    for i in range(REPLAYS):
        if i > 0:                                      # eager work between replays
            q.copy_(dev(make_decode_inputs(case, seed=100 + i).q, case.dtype))
            lens = shorter_lengths(inp.seqlens_k, rng)
            sl.copy_(dev_i32(lens))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref_o = torch.empty_like(out)
        ref_l = torch.empty_like(lse)
        run(ref_o, ref_l, ws_eager)
        torch.cuda.synchronize()
        say(f"  replay {i}: lengths {lens.tolist()}")
        assert same_bits(out, ref_o) and same_bits(lse, ref_l), f"replay {i} differs from the eager call"
        if i in (0, REPLAYS - 1):
            cur = dataclasses.replace(inp, q=inp.q if i == 0 else make_decode_inputs(case, seed=100 + i).q,
                                      seqlens_k=lens)
            Oref, lref = oracle_decode(cur)
            assert max_abs_err(to_f64(out), Oref) <= TOL[case.dtype]
            L = to_f64(lse)
            assert (np.isneginf(L) == np.isneginf(lref)).all()


def test_prefill_graph_replays():
    from attention_forward_tiled_amd import attn_prefill_fwd
    case = PrefillCase("graph_f16_d128_causal_paged", 2, 8, 2, 300, 700, 128, "f16", True, "paged",
                       seqlens_k=(700, 450))
    say(f"prefill graph capture, {case}")
    inp = make_prefill_inputs(case, seed=22)
    q = dev(inp.q, case.dtype)
    k, v = dev(inp.k, case.dtype), dev(inp.v, case.dtype)
    bt, sl = dev_i32(inp.block_table), dev_i32(inp.seqlens_k)

    def run(o, lse):
        attn_prefill_fwd(q, k, v, causal=True, block_table=bt, seqlens_k=sl, seqlen_k=case.seqlen_k,
                         out=o, lse=lse)

    out = torch.empty_like(q)
    lse = torch.empty((case.batch, case.heads_q, case.seqlen_q), dtype=torch.float32, device="cuda")
    run(out, lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(out, lse)
    torch.cuda.synchronize()

    rng = np.random.default_rng(8)
    lens, qbits = inp.seqlens_k, inp.q
    for i in range(REPLAYS):
        if i > 0:
            qbits = make_prefill_inputs(case, seed=200 + i).q
            q.copy_(dev(qbits, case.dtype))
            lens = shorter_lengths(inp.seqlens_k, rng)
            sl.copy_(dev_i32(lens))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref_o, ref_l = torch.empty_like(out), torch.empty_like(lse)
        run(ref_o, ref_l)
        torch.cuda.synchronize()
        say(f"  replay {i}: lengths {lens.tolist()}")
        assert same_bits(out, ref_o) and same_bits(lse, ref_l), f"replay {i} differs from the eager call"
        if i in (0, REPLAYS - 1):
            Oref, lref = oracle.attention(bits_to_f64(qbits, case.dtype), bits_to_f64(inp.k, case.dtype),
                                          bits_to_f64(inp.v, case.dtype), causal=True,
                                          block_table=inp.block_table, seqlens_k=lens)
            assert max_abs_err(to_f64(out), Oref) <= tolerance(case)
            assert (np.isneginf(to_f64(lse)) == np.isneginf(lref)).all()


def test_packed_prefill_graph_new_offsets():
    """Packed queries: the per-sequence split of a fixed total_q changes between replays."""
    from attention_forward_tiled_amd import attn_prefill_fwd
    case = PrefillCase("graph_bf16_d64_packed", 3, 4, 2, 300, 600, 64, "bf16", True, "paged",
                       seqlens_k=(600, 300, 450))
    say(f"packed prefill graph capture, {case}")
    inp = make_prefill_inputs(case, seed=23)
    splits = [(100, 200, 0), (300, 0, 0), (1, 150, 149), (0, 0, 300)]
    total = 300
    q = dev(np.ascontiguousarray(inp.q[0]), case.dtype)          # [total, Hq, d]
    k, v = dev(inp.k, case.dtype), dev(inp.v, case.dtype)
    bt, sl = dev_i32(inp.block_table), dev_i32(inp.seqlens_k)
    cu = dev_i32(np.concatenate([[0], np.cumsum(splits[0])]))

    def run(o, lse):
        attn_prefill_fwd(q, k, v, causal=True, block_table=bt, seqlens_k=sl, seqlen_k=case.seqlen_k,
                         cu_seqlens_q=cu, max_seqlen_q=total, out=o, lse=lse)

    out = torch.empty_like(q)
    lse = torch.empty((case.heads_q, total), dtype=torch.float32, device="cuda")
    run(out, lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(out, lse)
    torch.cuda.synchronize()

    qf = bits_to_f64(inp.q[0], case.dtype)
    kf, vf = bits_to_f64(inp.k, case.dtype), bits_to_f64(inp.v, case.dtype)
    for i, qlens in enumerate(splits):
        cuh = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
        cu.copy_(dev_i32(cuh))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref_o, ref_l = torch.empty_like(out), torch.empty_like(lse)
        run(ref_o, ref_l)
        torch.cuda.synchronize()
        say(f"  replay {i}: query counts {qlens}")
        assert same_bits(out, ref_o) and same_bits(lse, ref_l), f"replay {i} differs from the eager call"
        O = to_f64(out)
        for b, n in enumerate(qlens):
            if n == 0:
                continue
            rows = slice(int(cuh[b]), int(cuh[b + 1]))
            Oref, _ = oracle.attention(qf[None, rows], kf, vf, causal=True,
                                       block_table=inp.block_table[b:b + 1], seqlens_k=inp.seqlens_k[b:b + 1])
            assert max_abs_err(O[rows], Oref[0]) <= tolerance(case)


def test_prefill_tail_split_graph_replays():
    """A tail-split call (main items, split units, combine: three kernels) with its
    workspace passed in, captured once and replayed with new queries and key lengths."""
    from attention_forward_tiled_amd import attn_prefill_fwd, attn_prefill_workspace_bytes
    case = PrefillCase("graph_bf16_d128_split_paged", 2, 8, 2, 300, 900, 128, "bf16", False, "paged",
                       seqlens_k=(900, 640))
    say(f"prefill tail-split graph capture, {case}")
    inp = make_prefill_inputs(case, seed=24)
    q = dev(inp.q, case.dtype)
    k, v = dev(inp.k, case.dtype), dev(inp.v, case.dtype)
    bt, sl = dev_i32(inp.block_table), dev_i32(inp.seqlens_k)
    need = attn_prefill_workspace_bytes(q, num_heads_kv=case.heads_kv, seqlen_k=case.seqlen_k, causal=False,
                                        kv_splits=4)
    assert need > 0, "the launch does not split"
    ws, ws_eager = (torch.empty(need, dtype=torch.uint8, device="cuda") for _ in range(2))

    def run(o, lse, w):
        attn_prefill_fwd(q, k, v, causal=False, block_table=bt, seqlens_k=sl, seqlen_k=case.seqlen_k,
                         out=o, lse=lse, kv_splits=4, workspace=w)

    out = torch.empty_like(q)
    lse = torch.empty((case.batch, case.heads_q, case.seqlen_q), dtype=torch.float32, device="cuda")
    run(out, lse, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(out, lse, ws)
    torch.cuda.synchronize()

    rng = np.random.default_rng(9)
    lens, qbits = inp.seqlens_k, inp.q
    for i in range(REPLAYS):
        if i > 0:
            qbits = make_prefill_inputs(case, seed=300 + i).q
            q.copy_(dev(qbits, case.dtype))
            lens = shorter_lengths(inp.seqlens_k, rng)
            sl.copy_(dev_i32(lens))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref_o, ref_l = torch.empty_like(out), torch.empty_like(lse)
        run(ref_o, ref_l, ws_eager)
        torch.cuda.synchronize()
        say(f"  replay {i}: lengths {lens.tolist()}")
        assert same_bits(out, ref_o) and same_bits(lse, ref_l), f"replay {i} differs from the eager call"
        if i in (0, REPLAYS - 1):
            Oref, lref = oracle.attention(bits_to_f64(qbits, case.dtype), bits_to_f64(inp.k, case.dtype),
                                          bits_to_f64(inp.v, case.dtype), causal=False,
                                          block_table=inp.block_table, seqlens_k=lens)
            assert max_abs_err(to_f64(out), Oref) <= tolerance(case)
            assert (np.isneginf(to_f64(lse)) == np.isneginf(lref)).all()
