"""A seeded sweep of random small shapes against the fp64 oracle.

The named cases elsewhere pin each launch form and edge case on purpose; this sweep
draws the arguments independently (head size, dtypes, mask, paged or dense K/V,
layout, GQA ratio, query and key counts, ragged key lengths, fp32 output, the precise
mode, the tail-split setting; packed queries; decode batches and split counts), so
that combinations nobody listed (and the launch form the host picks for them) meet
the oracle too. Sizes stay small enough for the oracle to finish each case in about
a second. Every draw is a pure function of its index, so a failure names a case that
can be rebuilt exactly."""
import numpy as np
import pytest
import torch

import oracle
from attn_workloads import DecodeCase, PrefillCase, bits_to_f64, make_decode_inputs, make_prefill_inputs
from gpu_util import (TOL, dev, dev_i32, gpu_prefill, lse_tolerance, max_abs_err, oracle_decode,
                      oracle_prefill, say, to_f64, tolerance)



def gpu(f):
    return pytest.mark.gpu(pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")(f))


PAIRS_CAP = 12_000_000     # B * Hq * S_q * S_k: about a second of oracle time at d = 256
N_PREFILL, N_PACKED, N_DECODE = 96, 24, 48


def draw_prefill(i: int):
    """Case i of the prefill sweep and its kv_splits argument."""
    rng = np.random.default_rng([2024, i])
    d = int(rng.choice([64, 128, 256]))
    dtype = str(rng.choice(["f16", "bf16"]))
    causal = bool(rng.integers(2))
    kv = str(rng.choice(["paged", "dense"]))
    layout = str(rng.choice(["bshd", "bhsd"]))
    hkv = int(rng.choice([1, 2, 3]))
    hq = hkv * int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
    B = int(rng.integers(1, 4))
    sk = int(rng.integers(1, 1300))
    sq = int(rng.integers(1, 700))
    if causal and rng.random() < 0.7:
        sq = min(sq, sk)                 # mostly chunked prefill; sometimes more queries than keys
    sq = max(1, min(sq, PAIRS_CAP // (B * hq * sk)))
    lens = None
    if kv == "paged" or rng.random() < 0.5:
        lens = tuple(int(x) for x in rng.integers(0, sk + 1, size=B))
        lens = (sk,) + lens[1:]          # keep the longest sequence at seqlen_k
        if B > 1 and rng.random() < 0.3:
            lens = lens[:-1] + (0,)          # a sequence with no key
    precise = rng.random() < 0.15
    out = "f32" if precise or rng.random() < 0.2 else None
    u = rng.random()
    splits = 0 if u < 0.5 else (1 if u < 0.65 else int(rng.integers(2, 9)))
    name = (f"r{i}_{dtype}_d{d}_{'causal' if causal else 'full'}_{kv}_{layout}_b{B}_h{hq}x{hkv}"
            f"_q{sq}_k{sk}{'_precise' if precise else ''}{'_f32' if out else ''}_s{splits}")
    return PrefillCase(name, B, hq, hkv, sq, sk, d, dtype, causal, kv, layout=layout, out_dtype=out,
                       precise=precise, seqlens_k=lens), splits


@gpu
@pytest.mark.parametrize("i", range(N_PREFILL))
def test_random_prefill(i):
    case, splits = draw_prefill(i)
    say(f"random prefill {case.name}")
    inp = make_prefill_inputs(case, seed=100 + i)
    O, lse = gpu_prefill(inp, with_lse=True, kv_splits=splits)
    Oref, lref = oracle_prefill(inp)
    err = max_abs_err(O, Oref)
    say(f"  max abs err {err:.3e} (tol {tolerance(case)})")
    assert err <= tolerance(case)
    fin = np.isfinite(lref)
    assert (np.isneginf(lse) == ~fin).all()
    assert np.abs(lse[fin] - lref[fin]).max(initial=0.0) <= lse_tolerance(case.dtype, case.precise)


def draw_packed(i: int):
    """Case i of the packed-query sweep (BSHD only) and each sequence's query count."""
    rng = np.random.default_rng([2025, i])
    d = int(rng.choice([64, 128, 256]))
    dtype = str(rng.choice(["f16", "bf16"]))
    causal = bool(rng.integers(2))
    kv = str(rng.choice(["paged", "dense"]))
    hkv = int(rng.choice([1, 2, 4]))
    hq = hkv * int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(2, 5))
    sk = int(rng.integers(64, 1100))
    sq = int(rng.integers(1, 500))
    sq = max(1, min(sq, PAIRS_CAP // (B * hq * sk)))
    lens = tuple(int(x) for x in rng.integers(0, sk + 1, size=B))
    q_lens = tuple(int(x) for x in rng.integers(0, sq + 1, size=B))
    q_lens = (sq,) + q_lens[1:]          # the host-side maximum is reached
    name = f"p{i}_{dtype}_d{d}_{'causal' if causal else 'full'}_{kv}_b{B}_h{hq}x{hkv}_q{q_lens}_k{lens}"
    return PrefillCase(name, B, hq, hkv, sq, sk, d, dtype, causal, kv, seqlens_k=lens), q_lens


@gpu
@pytest.mark.parametrize("i", range(N_PACKED))
def test_random_packed_prefill(i):
    from attention_forward_tiled_amd import attn_prefill_fwd
    c, q_lens = draw_packed(i)
    say(f"random packed prefill {c.name}")
    inp = make_prefill_inputs(c, seed=200 + i)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = dev(np.concatenate([inp.q[b, :n] for b, n in enumerate(q_lens)], axis=0), c.dtype)
    bt = dev_i32(inp.block_table) if inp.block_table is not None else None
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full((c.heads_q, int(cu[-1])), float("nan"), dtype=torch.float32, device="cuda")
    attn_prefill_fwd(q, dev(inp.k, c.dtype), dev(inp.v, c.dtype), causal=c.causal, block_table=bt,
                     seqlens_k=dev_i32(inp.seqlens_k), seqlen_k=c.seqlen_k, cu_seqlens_q=dev_i32(cu),
                     max_seqlen_q=c.seqlen_q, out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    O, L = to_f64(out), to_f64(lse)
    qf, kf, vf = (bits_to_f64(x, c.dtype) for x in (inp.q, inp.k, inp.v))
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
        assert max_abs_err(O[rows], Oref[0]) <= tolerance(c), b
        lg, lr = L[:, rows], lref[0]
        fin = np.isfinite(lr)
        assert (np.isneginf(lg) == ~fin).all(), b
        assert np.abs(lg[fin] - lr[fin]).max(initial=0.0) <= lse_tolerance(c.dtype), b


def draw_decode(i: int):
    rng = np.random.default_rng([2026, i])
    d = int(rng.choice([64, 128, 256]))
    dtype = str(rng.choice(["f16", "bf16"]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    hq = hkv * int(rng.choice([1, 2, 3, 4, 8, 16]))
    B = int(rng.integers(1, 9))
    top = int(rng.choice([64, 700, 3000, 9000]))
    lens = tuple(int(x) for x in rng.integers(0, top + 1, size=B))
    if B > 1 and rng.random() < 0.3:
        lens = (0,) + lens[1:]               # a sequence with no key
    lens = lens if max(lens) > 0 else (1,) + lens[1:]
    splits = int(rng.choice([1, 2, 3, 7, 16, 64]))
    name = f"d{i}_{dtype}_d{d}_b{B}_h{hq}x{hkv}_max{max(lens)}_s{splits}"
    return DecodeCase(name, B, hq, hkv, d, dtype, lengths_fixed=lens), splits


@gpu
@pytest.mark.parametrize("i", range(N_DECODE))
def test_random_decode(i):
    from test_decode_gpu import gpu_decode
    case, splits = draw_decode(i)
    say(f"random decode {case.name}")
    inp = make_decode_inputs(case, seed=300 + i)
    O, lse = gpu_decode(inp, splits, with_lse=True)
    Oref, lref = oracle_decode(inp)
    err = max_abs_err(O, Oref)
    say(f"  max abs err {err:.3e}")
    assert err <= TOL[case.dtype]
    fin = np.isfinite(lref)
    assert (np.isneginf(lse) == ~fin).all()
    assert np.abs(lse[fin] - lref[fin]).max(initial=0.0) <= lse_tolerance(case.dtype)


def test_draws_cover_the_argument_space():
    # (CPU) the sweep is only useful if its draws reach every value of every argument
    pre = [draw_prefill(i) for i in range(N_PREFILL)]
    cs = [c for c, _ in pre]
    assert {c.head_dim for c in cs} == {64, 128, 256}
    assert {c.dtype for c in cs} == {"f16", "bf16"} and {c.causal for c in cs} == {True, False}
    assert {c.kv for c in cs} == {"paged", "dense"} and {c.layout for c in cs} == {"bshd", "bhsd"}
    assert any(c.precise for c in cs) and any(c.out_dtype == "f32" and not c.precise for c in cs)
    assert {s for _, s in pre} >= {0, 1} and any(s >= 2 for _, s in pre)
    assert any(c.causal and c.seqlen_q > min(c.lengths()) for c in cs)
    assert any(0 in c.lengths() for c in cs)
    dec = [draw_decode(i) for i in range(N_DECODE)]
    assert {c.head_dim for c, _ in dec} == {64, 128, 256}
    assert any(0 in c.lengths_fixed for c, _ in dec) and {s for _, s in dec} >= {1, 64}
