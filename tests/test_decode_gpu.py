"""GPU parity of the split-KV decode (attn_decode_fwd) and the standalone
log-sum-exp combine (attn_splitkv_combine) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from attn_workloads import CONFIGS, DecodeCase, make_decode_inputs
from gpu_util import (TOL, check_bf16_rounding, dev, dev_i32, lse_tolerance, max_abs_err, oracle_decode, say,
                      to_f64)
from oracle.rounding import round_bf16

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def gpu_decode(inp, num_splits, out_dtype=None, with_lse=False, out_round="rtne"):
    """attn_decode_fwd on the seeded inputs. The output and lse buffers are NaN-filled
    before the call and must come back written (O finite, lse never NaN)."""
    from attention_forward_tiled_amd import attn_decode_fwd
    c = inp.case
    lse = torch.full((c.batch, c.heads_q), float("nan"), device="cuda") if with_lse else None
    out = torch.full((c.batch, c.heads_q, c.head_dim), float("nan"),
                     dtype={"bf16": torch.bfloat16, "f16": torch.float16}[c.dtype] if out_dtype is None
                     else out_dtype, device="cuda")
    o = attn_decode_fwd(dev(inp.q, c.dtype), dev(inp.k_cache, c.dtype), dev(inp.v_cache, c.dtype),
                        dev_i32(inp.block_table), dev_i32(inp.seqlens_k),
                        max_seqlen_k=inp.max_seqlen_k, num_splits=num_splits,
                        out=out, lse=lse, out_round=out_round)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()), "decode output left unwritten (NaN) or non-finite"
    if lse is not None:
        assert not bool(torch.isnan(lse).any()), "decode lse left unwritten"
    return to_f64(o), (to_f64(lse) if with_lse else None)




SMALL = [
    (DecodeCase("bf16_g4_d128", 5, 8, 2, 128, "bf16", lengths_fixed=(1, 63, 64, 65, 1000)), (1, 3, 16)),
    (DecodeCase("f16_g1_d128", 4, 4, 4, 128, "f16", lengths_fixed=(700, 129, 4096, 5)), (1, 7)),
    (DecodeCase("bf16_g8_d64", 3, 16, 2, 64, "bf16", lengths_fixed=(333, 64, 2000)), (2, 16)),
    (DecodeCase("f16_g16_d128", 2, 32, 2, 128, "f16", lengths_fixed=(1500, 257)), (4,)),
    (DecodeCase("bf16_g2_d256", 3, 4, 2, 256, "bf16", lengths_fixed=(900, 1, 190)), (1, 5)),
    (DecodeCase("f16_g3_d128", 2, 6, 2, 128, "f16", lengths_fixed=(640, 641)), (10,)),
]


@pytest.mark.parametrize("case,splits", SMALL, ids=lambda x: getattr(x, "name", str(x)))
def test_decode_small(case, splits):
    inp = make_decode_inputs(case, seed=5)
    Oref, lref = oracle_decode(inp)
    for s in splits:
        say(f"decode parity {case} num_splits={s}")
        O, lse = gpu_decode(inp, s, with_lse=True)
        err = max_abs_err(O, Oref)
        say(f"  max abs err {err:.3e}")
        assert err <= TOL[case.dtype]
        assert np.abs(lse - lref).max() <= lse_tolerance(case.dtype)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("splits", [1, 4, 16])
def test_decode_empty_sequences(splits, d):
    # sequences with no key (reading: O = 0, lse = -inf) next to ordinary ones; the
    # balanced split kernel never visits them, the combine writes their rows
    case = DecodeCase("bf16_empty", 5, 8, 2, d, "bf16", lengths_fixed=(0, 300, 0, 5000, 64))
    inp = make_decode_inputs(case, seed=8)
    Oref, lref = oracle_decode(inp)
    say(f"decode with empty sequences d={d} num_splits={splits}")
    O, lse = gpu_decode(inp, splits, with_lse=True)
    assert max_abs_err(O, Oref) <= TOL[case.dtype]
    empty = inp.seqlens_k == 0
    assert (O[empty] == 0).all() and np.isneginf(lse[empty]).all() and np.isneginf(lref[empty]).all()
    assert np.abs(lse[~empty] - lref[~empty]).max() <= lse_tolerance(case.dtype)


def test_decode_many_short_sequences():
    # many sequences shorter than a workgroup's page range: ranges span several runs
    lens = tuple(int(x) for x in np.random.default_rng(3).integers(1, 700, size=48))
    case = DecodeCase("f16_many_short", 48, 8, 8, 64, "f16", lengths_fixed=lens)
    inp = make_decode_inputs(case, seed=9)
    Oref, lref = oracle_decode(inp)
    for s in (2, 16):
        say(f"decode many short sequences num_splits={s}")
        O, lse = gpu_decode(inp, s, with_lse=True)
        assert max_abs_err(O, Oref) <= TOL[case.dtype]
        assert np.abs(lse - lref).max() <= lse_tolerance(case.dtype)


@pytest.mark.parametrize("d", [128, 64])
def test_decode_split_count_invariance(d):
    # other split counts move the partition ends (and, at d = 64, which pages share a
    # barrier); the results agree to within fp32 rounding of the merges
    case = DecodeCase("inv", 3, 8, 2, d, "bf16", lengths_fixed=(3000, 64, 1777))
    inp = make_decode_inputs(case, seed=6)
    outs = []
    for s in (1, 2, 3, 16, 64):
        say(f"decode split invariance d={d} num_splits={s}")
        outs.append(gpu_decode(inp, s, out_dtype=torch.float32)[0])
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2e-2


@pytest.mark.parametrize("d", [128, 64])
def test_named_decode_full(d):
    # Full size, every sequence and head against the oracle (run one sequence at a time
    # to bound host memory), in the launch configuration the benchmark times.
    case = CONFIGS["splitkv_decode_bf16_64k"].with_(head_dim=d)
    say(f"decode parity (full size, all sequences) {case.name} d={d}")
    inp = make_decode_inputs(case, seed=0)
    O, lse = gpu_decode(inp, case.num_splits, with_lse=True)
    Oref, lref = oracle_decode(inp, per_call=1)
    err = max_abs_err(O, Oref)
    lerr = float(np.abs(lse - lref).max())
    say(f"  max abs err {err:.3e}, lse err {lerr:.3e} over all {case.batch} sequences "
        f"(lengths {int(inp.seqlens_k.min())}..{int(inp.seqlens_k.max())})")
    assert err <= TOL[case.dtype]
    assert lerr <= lse_tolerance(case.dtype)


@pytest.mark.parametrize("d", [128, 64])
def test_decode_deterministic(d):
    case = DecodeCase("det", 4, 32, 8, d, "bf16", lengths_fixed=(5000, 20000, 64, 1))
    inp = make_decode_inputs(case, seed=7)
    say(f"decode determinism d={d}")
    a, _ = gpu_decode(inp, 16)
    b, _ = gpu_decode(inp, 16)
    np.testing.assert_array_equal(a, b)


def _partials(seed, B=3, H=5, S=7, d=128):
    rng = np.random.default_rng(seed)
    po = rng.standard_normal((B, H, S, d)).astype(np.float32)
    pl = (rng.standard_normal((B, H, S)) * 20).astype(np.float32)
    pl[0, 0, :] = -np.inf                 # every split empty
    pl[0, 1, 1:] = -np.inf                # a single non-empty split
    pl[1, 2, ::2] = -np.inf
    pl[2, 3, 3] = 80.0                    # one split dominates
    po[np.isneginf(pl)] = np.nan          # an empty split's O_s must never be read
    return po, pl


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("odt", ["f32", "bf16", "f16"])
def test_combine_against_formula(d, odt):
    from attention_forward_tiled_amd import attn_splitkv_combine
    say(f"combine parity d={d} out={odt}")
    po, pl = _partials(d, d=d)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[odt]
    lse = torch.empty(pl.shape[:2], device="cuda")
    o = attn_splitkv_combine(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(),
                             out_dtype=tdt, lse=lse)
    torch.cuda.synchronize()
    Oref, lref = oracle.lse_combine(po.astype(np.float64), pl.astype(np.float64))
    tol = {"f32": 1e-5, "bf16": 4e-2, "f16": 2e-2}[odt]
    assert max_abs_err(to_f64(o), Oref) <= tol
    L = to_f64(lse)
    assert np.isneginf(L[0, 0]) and np.isneginf(lref[0, 0])
    fin = np.isfinite(lref)
    assert np.abs(L[fin] - lref[fin]).max() <= 1e-4


@pytest.mark.parametrize("mode", ["rtne", "rtna", "rtz"])
def test_decode_bf16_output_rounding(mode):
    case = DecodeCase("bf16_round_dec", 4, 16, 4, 128, "bf16", lengths_fixed=(900, 64, 3000, 17))
    inp = make_decode_inputs(case, seed=12)
    say(f"decode bf16 output rounding {mode}")
    O, _ = gpu_decode(inp, 8, out_round=mode)
    O32, _ = gpu_decode(inp, 8, out_dtype=torch.float32)
    Oref, _ = oracle_decode(inp)
    assert max_abs_err(O, round_bf16(Oref, mode)) <= TOL[case.dtype]
    check_bf16_rounding(O, O32, mode)


@pytest.mark.parametrize("mode", ["rtna", "rtz"])
def test_combine_bf16_output_rounding(mode):
    from attention_forward_tiled_amd import attn_splitkv_combine
    say(f"combine bf16 output rounding {mode}")
    po, pl = _partials(77, d=128)
    a = torch.from_numpy(po).cuda()
    b = torch.from_numpy(pl).cuda()
    o = attn_splitkv_combine(a, b, out_dtype=torch.bfloat16, out_round=mode)
    o32 = attn_splitkv_combine(a, b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    Oref, _ = oracle.lse_combine(po.astype(np.float64), pl.astype(np.float64))
    assert max_abs_err(to_f64(o), round_bf16(Oref, mode)) <= 4e-2
    check_bf16_rounding(to_f64(o), to_f64(o32), mode)


def test_decode_long_context():
    # 256k and 128k-1 keys: 4096 pages per sequence and KV head, a ragged last page
    case = DecodeCase("bf16_long_context", 2, 8, 2, 128, "bf16", lengths_fixed=(262144, 131071))
    inp = make_decode_inputs(case, seed=10)
    Oref, lref = oracle_decode(inp)
    for s in (1, 16):
        say(f"decode long context num_splits={s}")
        O, lse = gpu_decode(inp, s, with_lse=True)
        assert max_abs_err(O, Oref) <= TOL[case.dtype]
        assert np.abs(lse - lref).max() <= lse_tolerance(case.dtype)


def test_decode_large_batch():
    # more sequences than the plan kernel has threads (several sequences per thread)
    lens = tuple(int(x) for x in np.random.default_rng(4).integers(0, 400, size=2500))
    case = DecodeCase("f16_large_batch", 2500, 4, 2, 64, "f16", lengths_fixed=lens)
    inp = make_decode_inputs(case, seed=11)
    Oref, lref = oracle_decode(inp)
    for s in (1, 8):
        say(f"decode large batch num_splits={s}")
        O, lse = gpu_decode(inp, s, with_lse=True)
        assert max_abs_err(O, Oref) <= TOL[case.dtype]
        fin = np.isfinite(lref)
        assert (np.isneginf(lse) == ~fin).all()
        assert np.abs(lse[fin] - lref[fin]).max() <= lse_tolerance(case.dtype)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("splits", [1, 16])
def test_decode_invalid_page_ids_are_left_out(splits, d):
    import dataclasses
    case = DecodeCase("bf16_bad_ids", 2, 8, 2, d, "bf16", lengths_fixed=(1000, 333))
    inp = make_decode_inputs(case, seed=15)
    nb = inp.k_cache.shape[0]
    bad = inp.block_table.copy()
    bad[0, 7] = nb + 1
    bad[1, 2] = -5
    say(f"decode with invalid page ids, d={d} num_splits={splits}")
    O, _ = gpu_decode(dataclasses.replace(inp, block_table=bad), splits)
    table = np.zeros_like(inp.block_table)
    keep0 = [j for j in range(16) if j != 7]
    keep1 = [j for j in range(6) if j != 2]
    table[0, :len(keep0)] = inp.block_table[0, keep0]
    table[1, :len(keep1)] = inp.block_table[1, keep1]
    ref = dataclasses.replace(inp, block_table=table, seqlens_k=np.array([1000 - 64, 333 - 64], dtype=np.int32))
    Oref, _ = oracle_decode(ref)
    assert max_abs_err(O, Oref) <= TOL[case.dtype]


@pytest.mark.parametrize("d", [128, 64])
def test_decode_growing_scores(d):
    # keys scaled up along each sequence (up to 12x at its end), so later pages keep
    # raising each row's maximum, at first by far more than 2^8 per page and later by
    # small steps: both the moves of the running reference and the pages that keep it
    # are exercised against the exact softmax
    import dataclasses
    from attn_workloads.generate import bits_to_f32, round_to_bits
    case = DecodeCase("bf16_ramp", 3, 8, 2, d, "bf16", lengths_fixed=(2000, 700, 4000))
    inp = make_decode_inputs(case, seed=21)
    k = bits_to_f32(inp.k_cache, "bf16")
    for b, L in enumerate(inp.seqlens_k.tolist()):
        for t in range(0, L, 64):
            n = min(64, L - t)
            ramp = 0.25 + 12.0 * ((t + np.arange(n)) / L) ** 2
            k[inp.block_table[b, t // 64], :n] *= ramp[:, None, None].astype(np.float32)
    grown = dataclasses.replace(inp, k_cache=round_to_bits(k, "bf16"))
    Oref, lref = oracle_decode(grown)
    for s in (1, 3, 16):
        say(f"decode growing scores d={d} num_splits={s}")
        O, lse = gpu_decode(grown, s, with_lse=True)
        err = max_abs_err(O, Oref)
        say(f"  max abs err {err:.3e}, lse err {np.abs(lse - lref).max():.3e}")
        assert err <= TOL[case.dtype]
        assert np.abs(lse - lref).max() <= lse_tolerance(case.dtype)
