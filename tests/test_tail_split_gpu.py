"""GPU parity of the prefill tail split: the key tiles of the last work items are given
to several workgroups whose fp32 partials the log-sum-exp combine merges (page "gfx942
unified attention, from the math up", section 8; the 7minutos.es article on MoonMath
AI's HIP attention kernel, paragraph "Punto de referencia"). Forced part counts on small
shapes (every item is then in the tail) against the fp64 oracle, O and lse; the
library's own choice on shapes whose last round is partly empty, in the four-wave, the
eight-wave and the d = 256 narrow forms, and on a causal launch with few items."""
import numpy as np
import pytest
import torch

import oracle
from attn_workloads import PrefillCase, bits_to_f64, make_prefill_inputs
from gpu_util import (check_bf16_rounding, dev, dev_i32, gpu_prefill, lse_tolerance, max_abs_err,
                      oracle_prefill, say, to_f64, tolerance)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

P = PrefillCase
FORCED = [
    (P("split_bf16_d128_dense_ragged", 1, 2, 2, 300, 1000, 128, "bf16", False, "dense"), 3),
    (P("split_f16_d64_gqa4_paged_empty_seq", 2, 8, 2, 200, 700, 64, "f16", False, "paged",
       seqlens_k=(700, 0)), 5),
    (P("split_bf16_d128_bhsd_f32out_empty_parts", 2, 4, 4, 130, 257, 128, "bf16", False, "dense",
       layout="bhsd", out_dtype="f32"), 7),
    (P("split_f16_d128_gqa8_64_parts", 1, 16, 2, 90, 150, 128, "f16", False, "paged"), 64),
    (P("split_bf16_d64_cross_ragged", 3, 4, 1, 333, 65, 64, "bf16", False, "dense",
       seqlens_k=(65, 1, 30)), 2),
    # d = 256: the eight-wave narrow kernel (16 rows per wave, 128 per item)
    (P("split_bf16_d256_dense_ragged", 2, 2, 2, 200, 700, 256, "bf16", False, "dense"), 3),
    (P("split_f16_d256_gqa2_paged_varlen_f32out", 2, 4, 2, 130, 500, 256, "f16", False, "paged",
       seqlens_k=(500, 64), out_dtype="f32"), 5),
    # causal launches with few items: every item split (bottom-right mask per part,
    # diagonal tiles in any part, rows whose keys all fall in other parts)
    (P("split_f16_d128_causal_chunk_paged", 2, 8, 2, 200, 700, 128, "f16", True, "paged",
       seqlens_k=(700, 300)), 3),
    (P("split_bf16_d64_causal_self_dense", 1, 4, 4, 300, 300, 64, "bf16", True, "dense"), 4),
    (P("split_bf16_d128_causal_gqa4_short_keys", 2, 16, 4, 90, 60, 128, "bf16", True, "paged",
       seqlens_k=(60, 0)), 2),
    (P("split_f16_d256_causal_chunk_gqa2", 2, 4, 2, 150, 600, 256, "f16", True, "paged",
       seqlens_k=(600, 200)), 3),
]


def _workspace_bytes(case, kv_splits):
    from attention_forward_tiled_amd import attn_prefill_workspace_bytes
    shape = ((case.batch, case.seqlen_q, case.heads_q, case.head_dim) if case.layout == "bshd"
             else (case.batch, case.heads_q, case.seqlen_q, case.head_dim))
    q = torch.empty(shape, dtype={"f16": torch.float16, "bf16": torch.bfloat16}[case.dtype], device="cuda")
    return attn_prefill_workspace_bytes(q, num_heads_kv=case.heads_kv, seqlen_k=case.seqlen_k,
                                        causal=case.causal, layout=case.layout, kv_splits=kv_splits)


@pytest.mark.parametrize("case,parts", FORCED, ids=lambda x: getattr(x, "name", str(x)))
def test_tail_split_forced(case, parts):
    say(f"tail split parity {case.name}, {parts} parts")
    assert _workspace_bytes(case, parts) > 0, "the launch does not split"
    inp = make_prefill_inputs(case, seed=5)
    O, lse = gpu_prefill(inp, with_lse=True, kv_splits=parts)
    Oref, lref = oracle_prefill(inp)
    err = max_abs_err(O, Oref)
    say(f"  max abs err {err:.3e} (tol {tolerance(case)})")
    assert err <= tolerance(case)
    fin = np.isfinite(lref)
    assert (np.isneginf(lse) == ~fin).all()
    assert np.abs(lse[fin] - lref[fin]).max(initial=0.0) <= lse_tolerance(case.dtype)
    # the same launch unsplit: both within the tolerance of the oracle, so within twice it
    # of each other; rows with no key are exactly zero in both
    O1, _ = gpu_prefill(inp, with_lse=True, kv_splits=1)
    assert max_abs_err(O, O1) <= 2 * tolerance(case)
    empty = ~fin if case.layout == "bhsd" else (~fin).transpose(0, 2, 1)    # over O's first 3 axes
    assert (O[empty] == 0).all() and (O1[empty] == 0).all()


@pytest.mark.parametrize("mode", ["rtne", "rtna", "rtz"])
def test_tail_split_bf16_output_rounding(mode):
    # the combine rounds the merged fp32 row: the bf16 output of a split launch relates to
    # the fp32 output of the same split launch as the rounding mode says
    case = P("split_bf16_d128_round", 2, 4, 2, 160, 600, 128, "bf16", False, "dense")
    say(f"tail split bf16 output rounding {mode}")
    inp = make_prefill_inputs(case, seed=6)
    O32, _ = gpu_prefill(inp, out_dtype="f32", kv_splits=4)
    O16, _ = gpu_prefill(inp, out_round=mode, kv_splits=4)
    check_bf16_rounding(O16, O32, mode)


def test_tail_split_packed_queries():
    from attention_forward_tiled_amd import attn_prefill_fwd
    case = P("split_bf16_d128_packed_gqa2", 3, 4, 2, 300, 800, 128, "bf16", False, "paged",
             seqlens_k=(800, 65, 300))
    q_lens = (300, 0, 129)
    say(f"tail split parity, packed queries {case.name} q_lens={q_lens}")
    inp = make_prefill_inputs(case, seed=7)
    c = case
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = dev(np.concatenate([inp.q[b, :n] for b, n in enumerate(q_lens)], axis=0), c.dtype)
    k, v = dev(inp.k, c.dtype), dev(inp.v, c.dtype)
    lse = torch.full((c.heads_q, int(cu[-1])), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
    attn_prefill_fwd(q, k, v, causal=False, block_table=dev_i32(inp.block_table),
                     seqlens_k=dev_i32(inp.seqlens_k), seqlen_k=c.seqlen_k, cu_seqlens_q=dev_i32(cu),
                     max_seqlen_q=c.seqlen_q, lse=lse, out=out, kv_splits=6)
    torch.cuda.synchronize()
    O, L = to_f64(out), to_f64(lse)
    assert np.isfinite(O).all() and not np.isnan(L).any()
    qf, kf, vf = (bits_to_f64(x, c.dtype) for x in (inp.q, inp.k, inp.v))
    for b, n in enumerate(q_lens):
        if n == 0:
            continue
        Oref, lref = oracle.attention(qf[b:b + 1, :n], kf, vf, causal=False,
                                      block_table=inp.block_table[b:b + 1], seqlens_k=inp.seqlens_k[b:b + 1])
        rows = slice(int(cu[b]), int(cu[b + 1]))
        err = max_abs_err(O[rows], Oref[0])
        say(f"  sequence {b}: {n} queries, max abs err {err:.3e}")
        assert err <= tolerance(case)
        assert np.abs(L[:, rows] - lref[0]).max() <= lse_tolerance(c.dtype)


def _sampled_check(case, inp, O, rows_of):
    """Oracle on chosen query rows of every (sequence, head) of a dense BSHD case."""
    inp_q, inp_k, inp_v, d, G = inp.q, inp.k, inp.v, case.head_dim, case.group
    worst = 0.0
    for b in range(case.batch):
        for h in range(case.heads_q):
            rows = rows_of(b, h)
            K = bits_to_f64(inp_k[b, :, h // G, :], case.dtype)
            V = bits_to_f64(inp_v[b, :, h // G, :], case.dtype)
            Oref, _ = oracle.attention_rows(bits_to_f64(inp_q[b, rows, h, :], case.dtype), K, V, rows,
                                            case.seqlen_k, case.seqlen_q, case.causal, 1.0 / np.sqrt(d))
            worst = max(worst, max_abs_err(O[b, rows, h, :], Oref))
    return worst


AUTO = [
    # four-wave form: 32 items of 128 rows, fewer than one round -> every item split
    P("auto_bf16_d128_s1024x4096", 1, 4, 4, 1024, 4096, 128, "bf16", False, "dense", poison=False),
    # eight-wave form: 17 KV heads x 64 query blocks = 1088 items of 256 rows, the last
    # 64 (one whole head) in a quarter-full round -> split
    P("auto_f16_d128_h17_s16384x2048_wg8", 1, 17, 17, 16384, 2048, 128, "f16", False, "dense", poison=False),
    # d = 256 narrow kernel: 5 heads x 64 query blocks = 320 items, the last 64 split
    P("auto_bf16_d256_h5_s8192x4096", 1, 5, 5, 8192, 4096, 256, "bf16", False, "dense", poison=False),
    # causal chunked prefill with few items: 2 x 4 KV heads x 8 blocks = 64 items, each split
    P("auto_bf16_d128_causal_chunk_256x4096", 2, 16, 4, 256, 4096, 128, "bf16", True, "dense", poison=False),
    P("auto_bf16_d256_causal_chunk_512x8192", 1, 16, 4, 512, 8192, 256, "bf16", True, "dense", poison=False),
]


@pytest.mark.parametrize("case", AUTO, ids=lambda c: c.name)
def test_tail_split_library_choice(case):
    say(f"tail split chosen by the library {case.name}")
    assert _workspace_bytes(case, 0) > 0, "the library does not split this launch"
    inp = make_prefill_inputs(case, seed=8)
    O, _ = gpu_prefill(inp, kv_splits=0)
    O1, _ = gpu_prefill(inp, kv_splits=1)
    diff = max_abs_err(O, O1)
    say(f"  split vs unsplit max abs diff {diff:.3e}")
    assert diff <= 2 * tolerance(case)
    rng = np.random.default_rng(8)
    S = case.seqlen_q
    # one seeded row per 32-row slice (every wave of every workgroup, split or not)
    worst = _sampled_check(case, inp, O, lambda b, h: np.minimum(
        np.arange(0, S, 32) + rng.integers(0, 32, -(-S // 32)), S - 1))
    say(f"  max abs err {worst:.3e} (tol {tolerance(case)})")
    assert worst <= tolerance(case)


POLICY = [
    # (case, splits?) for the library's own choice (kv_splits = 0) on 256 CUs
    (P("long_noncausal_bf16_s16384", 4, 16, 16, 16384, 16384, 128, "bf16", False, "dense"), False),  # 16 full rounds
    (P("gqa_causal_paged_f16_s2048", 1, 32, 8, 2048, 2048, 128, "f16", True, "paged"), False),      # paired form
    (P("chunked_prefill_bf16_512x4096", 4, 16, 4, 512, 4096, 128, "bf16", True, "paged"), False),   # one item per CU
    (P("causal_mha_bf16_d256_s4096", 2, 16, 16, 4096, 4096, 256, "bf16", True, "dense"), False),
    (P("tail_noncausal_bf16_h25_s16384", 1, 25, 25, 16384, 16384, 128, "bf16", False, "dense"), True),
    (P("chunked_small_bf16_2x256x4096", 2, 16, 4, 256, 4096, 128, "bf16", True, "paged"), True),
    (P("half_full_d64_round", 3, 6, 6, 8192, 8192, 64, "bf16", False, "dense"), False),  # every CU still busy
    (P("short_causal_chunks_2048", 1, 32, 8, 512, 2048, 128, "f16", True, "paged"), False),  # keys < 3072
    (P("short_noncausal_1024", 1, 4, 4, 1024, 1024, 128, "bf16", False, "dense"), False),   # keys < 2048
    (P("precise_noncausal", 1, 4, 4, 1024, 4096, 128, "f16", False, "dense", precise=True, out_dtype="f32"), False),
]


@pytest.mark.parametrize("case,splits", POLICY, ids=lambda x: getattr(x, "name", str(x)))
def test_tail_split_policy(case, splits):
    """Which launches the library splits by itself (the rule of the split planner)."""
    from attention_forward_tiled_amd import attn_device_info
    if attn_device_info(0)["compute_units"] != 256:
        pytest.skip("the rule is stated for 256 CUs")
    say(f"tail split policy {case.name}: expect {'split' if splits else 'no split'}")
    from attention_forward_tiled_amd import attn_prefill_workspace_bytes
    shape = ((case.batch, case.seqlen_q, case.heads_q, case.head_dim) if case.layout == "bshd"
             else (case.batch, case.heads_q, case.seqlen_q, case.head_dim))
    q = torch.empty(shape, dtype={"f16": torch.float16, "bf16": torch.bfloat16}[case.dtype], device="cuda")
    need = attn_prefill_workspace_bytes(q, num_heads_kv=case.heads_kv, seqlen_k=case.seqlen_k, causal=case.causal,
                                        layout=case.layout, precise=case.precise)
    assert (need > 0) == splits, need


BAD_ID_SPLIT = [
    (P("split_bf16_d128_paged_bad_ids", 2, 8, 2, 100, 640, 128, "bf16", False, "paged",
       seqlens_k=(640, 400)), 3),
    (P("split_f16_d256_paged_bad_ids", 2, 6, 2, 200, 640, 256, "f16", False, "paged",
       seqlens_k=(640, 400)), 4),
]


@pytest.mark.parametrize("case,parts", BAD_ID_SPLIT, ids=lambda x: getattr(x, "name", str(x)))
def test_tail_split_invalid_page_ids_are_left_out(case, parts):
    # a page id outside [0, num_blocks) drops that page's 64 keys in whichever part holds
    # it; non-causal, so the expected result is the oracle on the table without those pages
    import dataclasses
    inp = make_prefill_inputs(case, seed=15)
    nb = inp.k.shape[0]
    bad = inp.block_table.copy()
    bad[0, 3] = -1
    bad[1, 5] = nb + 7
    say(f"tail split parity with invalid page ids {case.name}, {parts} parts")
    O, _ = gpu_prefill(dataclasses.replace(inp, block_table=bad), kv_splits=parts)
    keep0 = [j for j in range(10) if j != 3]
    keep1 = [j for j in range(7) if j != 5]
    table = inp.block_table.copy()
    table[:2] = 0
    table[0, :len(keep0)] = inp.block_table[0, keep0]
    table[1, :len(keep1)] = inp.block_table[1, keep1]
    lens = inp.seqlens_k.copy()
    lens[:2] -= 64
    Oref, _ = oracle_prefill(dataclasses.replace(inp, block_table=table, seqlens_k=lens))
    err = max_abs_err(O, Oref)
    say(f"  max abs err {err:.3e}")
    assert err <= tolerance(case)
