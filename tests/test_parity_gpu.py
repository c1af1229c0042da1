"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Element-by-element max-abs error on the same seeded inputs, with the tolerances
fp16 2e-2, bf16 4e-2, and 1e-4 for the fp32-accumulated precise mode. Small
cases span several 64-key tiles and a ragged tail; the named workloads run at
full size in the launch configuration the benchmark times, the largest ones
checked on sampled outputs.
"""
import numpy as np
import pytest
import torch

import oracle
from attn_workloads import CONFIGS, PrefillCase, bits_to_f64, make_prefill_inputs
from gpu_util import (check_bf16_rounding, dev, dev_i32, gpu_prefill, lse_tolerance, max_abs_err,
                      oracle_prefill, say, to_f64, tolerance)
from oracle.rounding import round_bf16

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]



P = PrefillCase
SMALL = [
    P("f16_d64_causal_paged", 2, 4, 2, 200, 200, 64, "f16", True, "paged"),
    P("bf16_d64_causal_paged_chunked", 2, 4, 2, 70, 190, 64, "bf16", True, "paged"),
    P("f16_d128_causal_paged", 2, 8, 2, 130, 300, 128, "f16", True, "paged"),
    P("bf16_d128_causal_paged", 1, 8, 8, 257, 257, 128, "bf16", True, "paged"),
    P("f16_d256_causal_paged", 1, 2, 1, 150, 150, 256, "f16", True, "paged"),
    P("bf16_d256_noncausal_dense", 2, 2, 2, 70, 133, 256, "bf16", False, "dense"),
    P("bf16_d128_noncausal_dense_bhsd", 2, 4, 4, 100, 257, 128, "bf16", False, "dense", layout="bhsd"),
    P("f16_d128_noncausal_dense_cross", 1, 4, 2, 333, 65, 128, "f16", False, "dense"),
    P("f16_d64_causal_dense_bhsd", 2, 4, 1, 129, 129, 64, "f16", True, "dense", layout="bhsd"),
    P("bf16_sq1_noncausal_paged", 3, 8, 2, 1, 500, 128, "bf16", False, "paged"),
    P("f16_sq1_causal_paged", 3, 8, 2, 1, 77, 128, "f16", True, "paged"),
    P("f16_gqa3", 1, 6, 2, 100, 100, 128, "f16", True, "paged"),
    P("bf16_gqa8", 1, 16, 2, 90, 200, 128, "bf16", True, "paged"),
    P("bf16_gqa16", 1, 32, 2, 40, 128, 64, "bf16", True, "paged"),
    P("f16_ragged_lengths", 3, 4, 2, 100, 300, 128, "f16", True, "paged", seqlens_k=(300, 100, 37)),
    P("bf16_ragged_dense", 3, 4, 4, 64, 200, 128, "bf16", False, "dense", seqlens_k=(200, 1, 130)),
    P("f16_precise_d128", 1, 2, 1, 150, 150, 128, "f16", True, "paged", out_dtype="f32", precise=True),
    P("bf16_f32_out", 1, 2, 2, 96, 96, 128, "bf16", True, "paged", out_dtype="f32"),
    P("f16_d256_gqa3_causal_paged", 2, 6, 2, 190, 190, 256, "f16", True, "paged"),
    P("bf16_d256_ragged_dense_bhsd", 3, 4, 4, 130, 300, 256, "bf16", True, "dense", layout="bhsd",
      seqlens_k=(300, 64, 7)),
    P("bf16_d256_f32_out_cross", 1, 4, 1, 333, 1000, 256, "bf16", False, "paged", out_dtype="f32"),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c.name)
def test_prefill_small(case):
    say(f"prefill parity {case}")
    inp = make_prefill_inputs(case, seed=1)
    O, lse = gpu_prefill(inp, with_lse=True)
    Oref, lref = oracle_prefill(inp)
    err = max_abs_err(O, Oref)
    say(f"  max abs err {err:.3e} (tol {tolerance(case)})")
    assert err <= tolerance(case)
    fin = np.isfinite(lref)
    assert (np.isneginf(lse) == ~fin).all()
    assert np.abs(lse[fin] - lref[fin]).max() <= lse_tolerance(case.dtype, case.precise)


def test_prefill_rows_without_keys_are_zero():
    # causal with a key length shorter than S_q: the first rows see no key at all
    case = P("empty_rows", 1, 2, 1, 100, 100, 128, "f16", True, "paged", seqlens_k=(40,))
    say(f"prefill parity {case}")
    inp = make_prefill_inputs(case, seed=2)
    O, lse = gpu_prefill(inp, with_lse=True)
    Oref, lref = oracle_prefill(inp)
    assert (O[0, :60] == 0).all() and np.isneginf(lse[0, :, :60]).all()
    assert max_abs_err(O, Oref) <= tolerance(case)


def test_paged_equals_dense_bitwise():
    base = P("pd", 2, 8, 2, 200, 200, 128, "bf16", True, "paged")
    say(f"paged vs dense {base}")
    a, _ = gpu_prefill(make_prefill_inputs(base, seed=3))
    b, _ = gpu_prefill(make_prefill_inputs(base.with_(kv="dense"), seed=3))
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("name", ["tiny_causal_f16_d64", "gqa_causal_paged_f16_s2048",
                                  "chunked_prefill_bf16_512x4096", "chunked_small_bf16_2x256x4096"])
def test_named_prefill_full(name):
    # (the last runs the causal few-item split: 64 items over 8 key parts and the combine)
    case = CONFIGS[name]
    say(f"prefill parity (full output) {name}")
    inp = make_prefill_inputs(case, seed=0)
    O, _ = gpu_prefill(inp)
    Oref, _ = oracle_prefill(inp)
    err = max_abs_err(O, Oref)
    say(f"  max abs err {err:.3e} (tol {tolerance(case)})")
    assert err <= tolerance(case)


def _every_wave_check(case, seed=0):
    """Full-size launch; the whole output must be written (NaN-filled before the launch,
    checked finite in gpu_prefill); against the oracle, every (sequence, head) gets one
    seeded row in every 32-row slice of the query axis, so every wave of every workgroup
    is compared (32 query rows per wave in every launch form). Dense BSHD inputs."""
    inp = make_prefill_inputs(case, seed=seed)
    O, _ = gpu_prefill(inp)
    B, S, H, d, G = case.batch, case.seqlen_q, case.heads_q, case.head_dim, case.group
    rng = np.random.default_rng(seed)
    worst, n_rows = 0.0, 0
    for b in range(B):
        for h in range(H):
            rows = np.arange(0, S, 32) + rng.integers(0, 32, size=-(-S // 32))
            rows = np.minimum(rows, S - 1)
            rows[0], rows[-1] = 0, S - 1
            K = bits_to_f64(inp.k[b, :, h // G, :], case.dtype)
            V = bits_to_f64(inp.v[b, :, h // G, :], case.dtype)
            Oref, _ = oracle.attention_rows(bits_to_f64(inp.q[b, rows, h, :], case.dtype), K, V, rows,
                                            case.seqlen_k, S, case.causal, 1.0 / np.sqrt(d))
            worst = max(worst, max_abs_err(O[b, rows, h, :], Oref))
            n_rows += rows.size
    say(f"  max abs err {worst:.3e} over {n_rows} (b, h, row) triples")
    assert worst <= tolerance(case)


@pytest.mark.parametrize("name", ["long_noncausal_bf16_s16384", "causal_mha_bf16_d256_s4096",
                                  "causal_mha_f16_d64_s4096", "tail_noncausal_bf16_h25_s16384"])
def test_named_full_size_every_wave(name):
    # the long workload in the eight-wave form (4096 workgroups of 256 rows, 32768 rows
    # checked), the d = 256 and d = 64 causal workloads in their launch forms, and the
    # 25-head workload with its tail split (1536 items, then 64 items in 4 key parts)
    case = CONFIGS[name]
    say(f"prefill parity (one row per wave of every workgroup) {name}")
    _every_wave_check(case)


def test_prefill_deterministic():
    case = CONFIGS["gqa_causal_paged_f16_s2048"]
    say(f"determinism {case.name}")
    inp = make_prefill_inputs(case, seed=4)
    a, _ = gpu_prefill(inp)
    b, _ = gpu_prefill(inp)
    np.testing.assert_array_equal(a, b)


# Launch forms (d <= 128, a device with 256 compute units): at d = 128, non-causal launches
# with at least 256 eight-wave workgroups of 256 query rows, and causal ones with at least
# 384, take that form; otherwise causal launches of
# fewer than 2048 four-wave workgroups split each workgroup's key range over two groups
# (the small causal cases above), pairing a heavy and a light query block per workgroup
# from 512 query blocks on, and the rest run one four-wave group per workgroup. The paired
# cases below include an odd block count (a middle block alone).
PAIRED = [
    P("f16_d128_causal_paged_paired_odd", 1, 32, 8, 2080, 2080, 128, "f16", True, "paged"),
    P("bf16_d64_causal_paged_paired_chunked", 2, 32, 8, 1030, 1100, 64, "bf16", True, "paged",
      seqlens_k=(1100, 1057)),
]


@pytest.mark.parametrize("case", PAIRED, ids=lambda c: c.name)
def test_prefill_paired_sampled(case):
    say(f"prefill parity (paired query blocks, sampled rows) {case}")
    inp = make_prefill_inputs(case, seed=6)
    O, _ = gpu_prefill(inp)
    rows = np.unique(np.concatenate([[0, 31, 32, 63, 1023, 1024, 1055, case.seqlen_q - 1],
                                     np.random.default_rng(2).choice(case.seqlen_q, 24, replace=False)]))
    rows = rows[rows < case.seqlen_q]
    Oref, _ = oracle_prefill(inp, q_index=rows)
    err = max_abs_err(O[:, rows], Oref)
    say(f"  max abs err {err:.3e} over {rows.size} rows x all (b, h)")
    assert err <= tolerance(case)


# GQA ratios up to the supported 128: a four-wave item then holds 128 / G positions (one
# at G >= 65, with rows 96..127 unused at G = 96), an eight-wave one 256 / G, a narrow
# d = 256 one 128 / G; with a forced tail split in the four-wave form.
WIDE_GROUPS = [
    (P("bf16_d128_gqa128_causal_paged_two_groups", 1, 128, 1, 50, 300, 128, "bf16", True, "paged"), 0),
    (P("f16_d64_gqa96_noncausal_dense_wg4", 2, 192, 2, 40, 200, 64, "f16", False, "dense",
       seqlens_k=(200, 77)), 0),
    (P("bf16_d128_gqa64_noncausal_paged_split", 1, 128, 2, 33, 700, 128, "bf16", False, "paged"), 5),
    (P("bf16_d256_gqa64_causal_dense_narrow", 1, 128, 2, 30, 100, 256, "bf16", True, "dense"), 0),
    (P("f16_d128_gqa128_noncausal_paged_wg8", 1, 256, 2, 1024, 150, 128, "f16", False, "paged"), 0),
]


@pytest.mark.parametrize("case,splits", WIDE_GROUPS, ids=lambda x: getattr(x, "name", str(x)))
def test_prefill_wide_groups(case, splits):
    say(f"prefill parity {case} kv_splits={splits}")
    inp = make_prefill_inputs(case, seed=9)
    O, lse = gpu_prefill(inp, with_lse=True, kv_splits=splits)
    rows = np.arange(case.seqlen_q)
    if case.seqlen_q > 256:
        rows = np.unique(np.concatenate([[0, 1, 2, 3, case.seqlen_q - 2, case.seqlen_q - 1],
                                         np.random.default_rng(4).choice(case.seqlen_q, 26, replace=False)]))
    Oref, lref = oracle_prefill(inp, q_index=rows)
    O, lse = (O[:, :, rows], lse[:, :, rows]) if case.layout == "bhsd" else (O[:, rows], lse[:, :, rows])
    err = max_abs_err(O, Oref)
    say(f"  max abs err {err:.3e} over {rows.size} rows x all (b, h)")
    assert err <= tolerance(case)
    fin = np.isfinite(lref)
    assert (np.isneginf(lse) == ~fin).all()
    assert np.abs(lse[fin] - lref[fin]).max() <= lse_tolerance(case.dtype, case.precise)


EIGHT_WAVE = [
    P("f16_d128_gqa2_causal_paged_1024wg8", 4, 64, 32, 1024, 1024, 128, "f16", True, "paged"),
    P("bf16_d128_noncausal_dense_1024wg8", 8, 32, 8, 1000, 1100, 128, "bf16", False, "dense",
      seqlens_k=(1100, 1000, 999, 64, 1, 700, 1100, 130)),
    P("bf16_d128_gqa8_causal_paged_ragged_wg8", 2, 32, 4, 4100, 4100, 128, "bf16", True, "paged",
      seqlens_k=(4100, 3000)),
    P("f16_d128_noncausal_dense_bhsd_cross_wg8", 4, 16, 16, 4100, 333, 128, "f16", False, "dense",
      layout="bhsd"),
    # group sizes that leave rows of a 256-row workgroup unused (G = 3: 85 positions x 3
    # heads; G = 6: 42 x 6) and a narrow one (G = 32: 8 positions x 32 heads)
    P("bf16_d128_gqa3_causal_paged_wg8", 3, 12, 4, 8200, 8200, 128, "bf16", True, "paged",
      seqlens_k=(8200, 5000, 7777)),
    P("f16_d128_gqa6_noncausal_dense_wg8", 4, 24, 4, 5000, 700, 128, "f16", False, "dense"),
    P("bf16_d128_gqa32_causal_paged_wg8", 4, 64, 2, 1100, 1100, 128, "bf16", True, "paged"),
    # precise P (hi + lo products) with an fp32 output, in the eight-wave form
    P("f16_d128_precise_f32out_dense_wg8", 4, 16, 16, 4096, 4096, 128, "f16", False, "dense",
      out_dtype="f32", precise=True),
    # (not eight-wave) the same launch sizes at d = 64, which keeps four-wave blocks
    P("f16_d64_gqa2_causal_paged_1024wg4", 4, 64, 32, 1024, 1024, 64, "f16", True, "paged"),
    P("f16_d64_gqa6_noncausal_dense_wg4", 4, 24, 4, 5000, 700, 64, "f16", False, "dense"),
    P("f16_d64_precise_f32out_dense_wg4", 4, 16, 16, 4096, 4096, 64, "f16", False, "dense",
      out_dtype="f32", precise=True),
    # launches that take the eight-wave form with one (non-causal) or one and a half
    # (causal) workgroups per CU: 256, 384, 512 and 784 items
    P("bf16_d128_noncausal_dense_256items_wg8", 1, 16, 16, 4096, 4096, 128, "bf16", False, "dense"),
    P("bf16_d128_causal_paged_384items_wg8", 1, 32, 8, 3072, 3072, 128, "bf16", True, "paged"),
    P("f16_d128_causal_paged_ragged_512items_wg8", 2, 32, 8, 2048, 2048, 128, "f16", True, "paged",
      seqlens_k=(2048, 1500)),
    P("bf16_d128_gqa3_causal_paged_784items_wg8", 1, 48, 16, 4096, 4096, 128, "bf16", True, "paged"),
    # (not eight-wave) causal MHA below 8192 keys: four-wave blocks, sampled rows
    P("bf16_d128_causal_mha_dense_4k_wg4", 2, 32, 32, 4096, 4096, 128, "bf16", True, "dense"),
    P("bf16_d128_precise_f32out_paged_wg8", 2, 32, 8, 4096, 3000, 128, "bf16", False, "paged",
      out_dtype="f32", precise=True, seqlens_k=(3000, 1999)),
]


@pytest.mark.parametrize("case", EIGHT_WAVE, ids=lambda c: c.name)
def test_prefill_eight_wave_sampled(case):
    say(f"prefill parity (sampled rows) {case}")
    inp = make_prefill_inputs(case, seed=5)
    O, _ = gpu_prefill(inp)
    rows = np.unique(np.concatenate([[0, 31, 32, 63, 64, 127, 128, 255, 256, 1099, 1100, case.seqlen_q - 1],
                                     np.random.default_rng(1).choice(case.seqlen_q, 24, replace=False)]))
    rows = rows[rows < case.seqlen_q]
    Oref, _ = oracle_prefill(inp, q_index=rows)
    err = max_abs_err(O[:, :, rows] if case.layout == "bhsd" else O[:, rows], Oref)
    say(f"  max abs err {err:.3e} over {rows.size} rows x all (b, h)")
    assert err <= tolerance(case)


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("mode", ["rtne", "rtna", "rtz"])
def test_prefill_bf16_output_rounding(mode, d):
    # the three bf16 output modes of the MoonMath benchmark page: parity against the
    # oracle rounded in the same mode, and the rounding relations against the fp32
    # output of the same launch
    case = P("bf16_round", 2, 8, 2, 160, 300, d, "bf16", True, "paged")
    say(f"prefill bf16 output rounding {mode} d={d}")
    inp = make_prefill_inputs(case, seed=11)
    O, _ = gpu_prefill(inp, out_round=mode)
    O32, _ = gpu_prefill(inp, out_dtype="f32")
    Oref, _ = oracle_prefill(inp)
    assert max_abs_err(O, round_bf16(Oref, mode)) <= tolerance(case)
    ties = check_bf16_rounding(O, O32, mode)
    say(f"  {ties} exact ties among {O.size} outputs")


# Packed queries: sequences with their own query counts in one [total_q, Hq, d] buffer
# (cu_seqlens_q), each with the bottom-right causal offset L_b - S_q,b. The oracle runs
# sequence by sequence on the same seeded values (drawn padded to the longest sequence).
VARLEN = [
    (P("f16_d128_causal_paged_varlen", 4, 8, 2, 257, 1000, 128, "f16", True, "paged",
       seqlens_k=(300, 50, 200, 1000)), (100, 0, 257, 64)),
    (P("bf16_d64_noncausal_dense_varlen", 3, 4, 4, 200, 130, 64, "bf16", False, "dense",
       seqlens_k=(130, 7, 130)), (33, 200, 1)),
    (P("bf16_d128_causal_paged_gqa4_varlen", 3, 16, 4, 700, 900, 128, "bf16", True, "paged",
       seqlens_k=(900, 700, 333)), (700, 129, 333)),
    # d = 256 (eight waves of 16 rows): packed queries with GQA 2
    (P("bf16_d256_causal_paged_gqa2_varlen", 3, 4, 2, 300, 700, 256, "bf16", True, "paged",
       seqlens_k=(700, 65, 300)), (300, 1, 129)),
    # eight-wave form (max_seqlen_q 4096: 16 x 8 heads x 8 sequences = 1024 workgroups)
    (P("f16_d128_noncausal_dense_varlen_wg8", 8, 8, 8, 4096, 1000, 128, "f16", False, "dense",
       seqlens_k=(200, 64, 1, 130, 700, 5, 64, 999)), (4096, 0, 1, 255, 256, 257, 1000, 3000)),
]


@pytest.mark.parametrize("case,q_lens", VARLEN, ids=lambda x: getattr(x, "name", str(x)))
def test_prefill_packed_queries(case, q_lens):
    from attention_forward_tiled_amd import attn_prefill_fwd
    say(f"prefill parity, packed queries {case.name} q_lens={q_lens}")
    inp = make_prefill_inputs(case, seed=13)
    c = case
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q_packed = np.concatenate([inp.q[b, :n] for b, n in enumerate(q_lens)], axis=0)   # [total, Hq, d]
    q = dev(q_packed, c.dtype)
    k, v = dev(inp.k, c.dtype), dev(inp.v, c.dtype)
    bt = dev_i32(inp.block_table) if inp.block_table is not None else None
    lse = torch.full((c.heads_q, int(cu[-1])), float("nan"), dtype=torch.float32, device="cuda")
    o = attn_prefill_fwd(q, k, v, causal=c.causal, block_table=bt, seqlens_k=dev_i32(inp.seqlens_k),
                         seqlen_k=c.seqlen_k, cu_seqlens_q=dev_i32(cu), max_seqlen_q=c.seqlen_q, lse=lse)
    torch.cuda.synchronize()
    O, L = to_f64(o), to_f64(lse)
    qf = bits_to_f64(inp.q, c.dtype)
    kf, vf = bits_to_f64(inp.k, c.dtype), bits_to_f64(inp.v, c.dtype)
    for b, n in enumerate(q_lens):
        if n == 0:
            continue
        if inp.block_table is not None:
            Oref, lref = oracle.attention(qf[b:b + 1, :n], kf, vf, causal=c.causal,
                                          block_table=inp.block_table[b:b + 1], seqlens_k=inp.seqlens_k[b:b + 1])
        else:
            Oref, lref = oracle.attention(qf[b:b + 1, :n], kf[b:b + 1], vf[b:b + 1], causal=c.causal,
                                          seqlens_k=inp.seqlens_k[b:b + 1])
        rows = slice(int(cu[b]), int(cu[b + 1]))
        err = max_abs_err(O[rows], Oref[0])
        say(f"  sequence {b}: {n} queries, {int(inp.seqlens_k[b])} keys, max abs err {err:.3e}")
        assert err <= tolerance(case)
        lg, lr = L[:, rows], lref[0]
        fin = np.isfinite(lr)
        assert (np.isneginf(lg) == np.isneginf(lr)).all()
        assert np.abs(lg[fin] - lr[fin]).max(initial=0.0) <= lse_tolerance(case.dtype, case.precise)


def test_prefill_long_keys():
    # a short chunk of queries against 128k keys (2048 pages in the table), all rows checked
    case = P("bf16_d128_causal_paged_128k", 1, 8, 2, 100, 131072, 128, "bf16", True, "paged",
             seqlens_k=(131000,))
    say(f"prefill parity {case}")
    inp = make_prefill_inputs(case, seed=12)
    O, lse = gpu_prefill(inp, with_lse=True)
    Oref, lref = oracle_prefill(inp)
    err = max_abs_err(O, Oref)
    say(f"  max abs err {err:.3e}")
    assert err <= tolerance(case)
    assert np.abs(lse - lref).max() <= lse_tolerance(case.dtype, case.precise)


BAD_ID_CASES = [
    P("bf16_d128_noncausal_paged_bad_ids", 2, 8, 2, 100, 640, 128, "bf16", False, "paged",
      seqlens_k=(640, 400)),
    P("f16_d256_noncausal_paged_bad_ids", 2, 6, 2, 200, 640, 256, "f16", False, "paged",
      seqlens_k=(640, 400)),
    # eight-wave form: 32 x 8 heads x 4 sequences = 1024 workgroups
    P("f16_d128_noncausal_paged_bad_ids_wg8", 4, 8, 8, 8192, 640, 128, "f16", False, "paged",
      seqlens_k=(640, 400, 640, 64)),
    # d = 64 (four-wave blocks at any size)
    P("f16_d64_noncausal_paged_bad_ids_wg4", 4, 8, 8, 8192, 640, 64, "f16", False, "paged",
      seqlens_k=(640, 400, 640, 64)),
]


@pytest.mark.parametrize("case", BAD_ID_CASES, ids=lambda c: c.name)
def test_prefill_invalid_page_ids_are_left_out(case):
    # a page id outside [0, num_blocks) drops that page's 64 keys (no out-of-bounds read);
    # non-causal, so the expected result is the oracle on the table without those pages
    import dataclasses
    inp = make_prefill_inputs(case, seed=14)
    nb = inp.k.shape[0]
    bad = inp.block_table.copy()
    bad[0, 3] = -1
    bad[1, 5] = nb + 7
    say(f"prefill parity with invalid page ids {case}")
    O, _ = gpu_prefill(dataclasses.replace(inp, block_table=bad))
    keep0 = [j for j in range(10) if j != 3]
    keep1 = [j for j in range(7) if j != 5]
    table = inp.block_table.copy()
    table[:2] = 0
    table[0, :len(keep0)] = inp.block_table[0, keep0]
    table[1, :len(keep1)] = inp.block_table[1, keep1]
    lens = inp.seqlens_k.copy()
    lens[:2] -= 64
    Oref, _ = oracle_prefill(dataclasses.replace(inp, block_table=table, seqlens_k=lens))
    assert max_abs_err(O, Oref) <= tolerance(case)


# Keys scaled up along the sequence (up to 12x at its end): along a row's key tiles the
# maximum keeps rising, at first by far more than 2^8 per tile and later by small steps,
# so the lazily moved reference maximum, its per-lane check and the skipped rescales all
# meet the exact softmax. One case per launch form.
GROWING = [
    P("bf16_d128_gqa4_causal_growing_pairs", 1, 32, 8, 2048, 2048, 128, "bf16", True, "dense"),
    P("f16_d128_gqa4_causal_growing_two_groups", 1, 8, 2, 1000, 1000, 128, "f16", True, "dense"),
    P("bf16_d64_noncausal_growing_wg4", 2, 8, 2, 700, 900, 64, "bf16", False, "dense"),
    P("bf16_d128_noncausal_growing_wg8", 8, 32, 8, 1000, 1100, 128, "bf16", False, "dense"),
    P("bf16_d256_causal_growing_narrow", 2, 6, 2, 700, 700, 256, "bf16", True, "dense"),
]


@pytest.mark.parametrize("case", GROWING, ids=lambda c: c.name)
def test_prefill_growing_scores(case):
    import dataclasses
    from attn_workloads.generate import bits_to_f32, round_to_bits
    say(f"prefill growing scores {case}")
    inp = make_prefill_inputs(case, seed=23)
    ramp = (0.25 + 12.0 * (np.arange(case.seqlen_k) / case.seqlen_k) ** 2).astype(np.float32)
    k = bits_to_f32(inp.k, case.dtype) * ramp[None, :, None, None]
    grown = dataclasses.replace(inp, k=round_to_bits(k, case.dtype))
    O, lse = gpu_prefill(grown, with_lse=True)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 255, 256, case.seqlen_q - 1],
                                     np.random.default_rng(2).choice(case.seqlen_q, 40, replace=False)]))
    rows = rows[rows < case.seqlen_q]
    Oref, lref = oracle_prefill(grown, q_index=rows)
    err = max_abs_err(O[:, rows], Oref)
    lerr = np.abs(lse[:, :, rows] - lref).max()
    say(f"  max abs err {err:.3e}, lse err {lerr:.3e} over {rows.size} rows x all (b, h)")
    assert err <= tolerance(case)
    assert lerr <= lse_tolerance(case.dtype, case.precise)
