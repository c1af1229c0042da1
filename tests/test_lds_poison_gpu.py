"""Parity against the fp64 oracle with the LDS-poisoning debug build (libattn_poison.so:
the same kernels, compiled so that each fills its LDS with NaN bit patterns before its
first copy). Any read of LDS that no copy or store wrote would carry NaN into the output,
so these cases, one or more per launch form and path that leaves LDS partly unwritten
(ragged key tails, invalid page ids, empty sequences, the two-group merge, the tail split,
decode rings), pin that every value the kernels consume was written first."""
import dataclasses

import numpy as np
import pytest
import torch

from attention_forward_tiled_amd import _lib
from attn_workloads import DecodeCase, PrefillCase as P, make_decode_inputs, make_prefill_inputs
from gpu_util import (TOL, gpu_prefill, lse_tolerance, max_abs_err, oracle_decode, oracle_prefill, say,
                      tolerance)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def poison_lib():
    # built by attention_forward_tiled_amd.build next to libattn.so; missing is a failure
    return _lib.open_library(_lib.POISON_LIB_PATH)


@pytest.fixture
def use_poison(poison_lib, monkeypatch):
    monkeypatch.setattr(_lib, "_LIB", poison_lib)
    assert _lib.load() is poison_lib


PREFILL = [
    # (case, kv_splits): two-group causal (paged, ragged, GQA), four-wave non-causal,
    # d = 64, the narrow d = 256 kernel, BHSD layout, an empty sequence, the paired and
    # eight-wave forms (sampled rows), forced tail splits, the causal few-item split
    (P("poison_f16_d128_causal_paged", 2, 8, 2, 130, 300, 128, "f16", True, "paged"), 0),
    (P("poison_bf16_d128_noncausal_dense_ragged", 3, 4, 4, 64, 200, 128, "bf16", False, "dense",
       seqlens_k=(200, 1, 130)), 0),
    (P("poison_f16_d64_causal_paged", 2, 4, 2, 200, 200, 64, "f16", True, "paged"), 0),
    (P("poison_bf16_d256_causal_paged", 2, 6, 2, 190, 190, 256, "bf16", True, "paged"), 0),
    (P("poison_bf16_d256_noncausal_bhsd", 3, 4, 4, 130, 300, 256, "bf16", False, "dense",
       layout="bhsd"), 0),
    (P("poison_f16_d128_empty_seq", 2, 8, 2, 200, 700, 128, "f16", False, "paged",
       seqlens_k=(700, 0)), 0),
    (P("poison_f16_d128_paired", 1, 32, 8, 2080, 2080, 128, "f16", True, "paged"), 0),
    (P("poison_bf16_d128_wg8", 8, 32, 8, 1000, 1100, 128, "bf16", False, "dense",
       seqlens_k=(1100, 1000, 999, 64, 1, 700, 1100, 130)), 0),
    (P("poison_bf16_d128_split", 2, 8, 2, 300, 900, 128, "bf16", False, "paged",
       seqlens_k=(900, 640)), 4),
    (P("poison_f16_d256_split", 2, 4, 2, 130, 500, 256, "f16", False, "paged",
       seqlens_k=(500, 64)), 5),
    (P("poison_bf16_d128_causal_chunk_split", 2, 16, 4, 256, 4096, 128, "bf16", True, "paged",
       seqlens_k=(4096, 3000)), 0),
]


@pytest.mark.parametrize("case,splits", PREFILL, ids=lambda x: getattr(x, "name", str(x)))
def test_prefill_reads_only_written_lds(use_poison, case, splits):
    say(f"prefill parity, LDS poisoned {case} kv_splits={splits}")
    inp = make_prefill_inputs(case, seed=21)
    O, lse = gpu_prefill(inp, with_lse=True, kv_splits=splits)
    rows = np.arange(case.seqlen_q)
    if case.seqlen_q > 600:
        rows = np.unique(np.concatenate([[0, 31, 32, 63, 64, 127, 128, 255, 256, case.seqlen_q - 1],
                                         np.random.default_rng(5).choice(case.seqlen_q, 16, replace=False)]))
    Oref, lref = oracle_prefill(inp, q_index=rows)
    Os, ls = (O[:, :, rows] if case.layout == "bhsd" else O[:, rows]), lse[:, :, rows]
    err = max_abs_err(Os, Oref)
    say(f"  max abs err {err:.3e}")
    assert err <= tolerance(case)
    fin = np.isfinite(lref)
    assert (np.isneginf(ls) == ~fin).all()
    assert np.abs(ls[fin] - lref[fin]).max(initial=0.0) <= lse_tolerance(case.dtype)


def test_prefill_invalid_page_ids_read_only_written_lds(use_poison):
    case = P("poison_bf16_d128_bad_ids", 2, 8, 2, 100, 640, 128, "bf16", False, "paged", seqlens_k=(640, 400))
    inp = make_prefill_inputs(case, seed=22)
    nb = inp.k.shape[0]
    bad = inp.block_table.copy()
    bad[0, 3] = -1
    bad[1, 5] = nb + 7
    say(f"prefill parity with invalid page ids, LDS poisoned {case}")
    O, _ = gpu_prefill(dataclasses.replace(inp, block_table=bad))
    table = inp.block_table.copy()
    table[:2] = 0
    table[0, :9] = inp.block_table[0, [j for j in range(10) if j != 3]]
    table[1, :6] = inp.block_table[1, [j for j in range(7) if j != 5]]
    lens = inp.seqlens_k.copy()
    lens[:2] -= 64
    Oref, _ = oracle_prefill(dataclasses.replace(inp, block_table=table, seqlens_k=lens))
    assert max_abs_err(O, Oref) <= tolerance(case)


DECODE = [
    (DecodeCase("poison_bf16_g4_d128", 5, 8, 2, 128, "bf16", lengths_fixed=(1, 63, 64, 65, 1000)), (1, 16)),
    (DecodeCase("poison_bf16_g8_d64", 3, 16, 2, 64, "bf16", lengths_fixed=(333, 0, 2000)), (1, 16)),
    (DecodeCase("poison_bf16_g2_d256", 3, 4, 2, 256, "bf16", lengths_fixed=(900, 1, 190)), (1, 5)),
]


@pytest.mark.parametrize("case,splits", DECODE, ids=lambda x: getattr(x, "name", str(x)))
def test_decode_reads_only_written_lds(use_poison, case, splits):
    from test_decode_gpu import gpu_decode
    inp = make_decode_inputs(case, seed=23)
    Oref, lref = oracle_decode(inp)
    for s in splits:
        say(f"decode parity, LDS poisoned {case} num_splits={s}")
        O, lse = gpu_decode(inp, s, with_lse=True)
        err = max_abs_err(O, Oref)
        say(f"  max abs err {err:.3e}")
        assert err <= TOL[case.dtype]
        fin = np.isfinite(lref)
        assert (np.isneginf(lse) == ~fin).all()
        assert np.abs(lse[fin] - lref[fin]).max(initial=0.0) <= lse_tolerance(case.dtype)


@pytest.mark.parametrize("splits", [1, 16])
def test_decode_invalid_page_ids_read_only_written_lds(use_poison, splits):
    from test_decode_gpu import gpu_decode
    case = DecodeCase("poison_bf16_g4_d128_bad_ids", 3, 8, 2, 128, "bf16", lengths_fixed=(700, 300, 1500))
    inp = make_decode_inputs(case, seed=24)
    nb = inp.k_cache.shape[0]
    bad = inp.block_table.copy()
    bad[0, 2] = -5
    bad[2, 7] = nb + 3
    say(f"decode parity with invalid page ids, LDS poisoned, num_splits={splits}")
    O, _ = gpu_decode(dataclasses.replace(inp, block_table=bad), splits)
    table = inp.block_table.copy()
    lens = inp.seqlens_k.copy()
    for b, j in ((0, 2), (2, 7)):
        n = -(-int(lens[b]) // 64)
        keep = [x for x in range(n) if x != j]
        table[b, :len(keep)] = inp.block_table[b, keep]
        lens[b] -= 64
    Oref, _ = oracle_decode(dataclasses.replace(inp, block_table=table, seqlens_k=lens))
    assert max_abs_err(O, Oref) <= TOL[case.dtype]


@pytest.mark.parametrize("i", range(0, 96, 4))
def test_random_prefill_reads_only_written_lds(use_poison, i):
    # every fourth draw of the seeded random sweep, against the poisoned build
    from test_random_shapes_gpu import draw_prefill
    case, splits = draw_prefill(i)
    say(f"random prefill, LDS poisoned {case.name}")
    inp = make_prefill_inputs(case, seed=100 + i)
    O, lse = gpu_prefill(inp, with_lse=True, kv_splits=splits)
    Oref, lref = oracle_prefill(inp)
    assert max_abs_err(O, Oref) <= tolerance(case)
    fin = np.isfinite(lref)
    assert (np.isneginf(lse) == ~fin).all()
    assert np.abs(lse[fin] - lref[fin]).max(initial=0.0) <= lse_tolerance(case.dtype, case.precise)


@pytest.mark.parametrize("i", range(0, 48, 4))
def test_random_decode_reads_only_written_lds(use_poison, i):
    from test_decode_gpu import gpu_decode
    from test_random_shapes_gpu import draw_decode
    case, splits = draw_decode(i)
    say(f"random decode, LDS poisoned {case.name}")
    inp = make_decode_inputs(case, seed=300 + i)
    O, lse = gpu_decode(inp, splits, with_lse=True)
    Oref, lref = oracle_decode(inp)
    assert max_abs_err(O, Oref) <= TOL[case.dtype]
    fin = np.isfinite(lref)
    assert (np.isneginf(lse) == ~fin).all()
