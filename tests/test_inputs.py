"""Seeded input generators: determinism, rounding, page tables, poisoning (CPU)."""
import numpy as np
import torch

from attn_workloads import (CONFIGS, DecodeCase, PrefillCase, bits_to_f64, make_decode_inputs,
                            make_prefill_inputs, round_to_bits)

SMALL = PrefillCase("small", batch=2, heads_q=4, heads_kv=2, seqlen_q=70, seqlen_k=150,
                    head_dim=64, dtype="bf16", causal=True, kv="paged", table="random")


def test_prefill_deterministic_per_seed():
    a = make_prefill_inputs(SMALL, seed=3)
    b = make_prefill_inputs(SMALL, seed=3)
    c = make_prefill_inputs(SMALL, seed=4)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.block_table, b.block_table)):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a.q, c.q)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32) * 3
    # exact ties: low 16 bits 0x8000, both even and odd upper halves
    ties = (rng.integers(0, 1 << 6, 1000).astype(np.uint32) << 17 | 0x3F800000 | 0x8000)   # mantissa-only variation: finite
    ties2 = ties | (1 << 16)
    x = np.concatenate([x, ties.view(np.float32), ties2.view(np.float32),
                        np.array([0.0, -0.0, 1e-40, -1e-40, 3.4e38, np.inf, -np.inf], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(round_to_bits(x, "bf16"), want)


def test_f16_rounding_matches_torch():
    x = np.random.default_rng(1).standard_normal(100000).astype(np.float32) * 100
    want = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(round_to_bits(x, "f16"), want)


def test_bits_upcast_exact():
    x = np.random.default_rng(2).standard_normal(1000).astype(np.float32)
    for dt, tdt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        bits = round_to_bits(x, dt)
        want = torch.from_numpy(x).to(tdt).to(torch.float64).numpy()
        np.testing.assert_array_equal(bits_to_f64(bits, dt), want)


def test_paged_holds_the_dense_values():
    inp = make_prefill_inputs(SMALL, seed=5)
    dense = make_prefill_inputs(SMALL.with_(kv="dense"), seed=5)
    tbl = inp.block_table
    assert sorted(tbl.ravel().tolist()) == list(range(tbl.size))      # a permutation of pages
    for b in range(SMALL.batch):
        for j in range(SMALL.seqlen_k):
            np.testing.assert_array_equal(inp.k[tbl[b, j // 64], j % 64], dense.k[b, j])
            np.testing.assert_array_equal(inp.v[tbl[b, j // 64], j % 64], dense.v[b, j])
    np.testing.assert_array_equal(inp.q, dense.q)


def test_prefill_tail_slots_poisoned():
    inp = make_prefill_inputs(SMALL, seed=6)
    f = bits_to_f64(inp.k, "bf16")
    tail = SMALL.seqlen_k % 64
    for b in range(SMALL.batch):
        last = inp.block_table[b, -1]
        assert np.isnan(f[last, tail:]).all()
        assert np.isfinite(f[last, :tail]).all()


def test_bhsd_is_a_transpose():
    a = make_prefill_inputs(SMALL.with_(kv="dense"), seed=7)
    b = make_prefill_inputs(SMALL.with_(kv="dense", layout="bhsd"), seed=7)
    np.testing.assert_array_equal(b.q, a.q.transpose(0, 2, 1, 3))
    np.testing.assert_array_equal(b.k, a.k.transpose(0, 2, 1, 3))


def test_decode_inputs_structure():
    case = DecodeCase("d", batch=6, heads_q=8, heads_kv=2, head_dim=64, len_lo=1, len_hi=300)
    inp = make_decode_inputs(case, seed=1)
    lens = inp.seqlens_k
    assert ((lens >= 1) & (lens <= 300)).all()
    pages = [-(-int(L) // 64) for L in lens]
    used = np.concatenate([inp.block_table[b, :n] for b, n in enumerate(pages)])
    assert len(set(used.tolist())) == used.size == sum(pages) == inp.k_cache.shape[0]
    kf = bits_to_f64(inp.k_cache, "bf16")
    for b, L in enumerate(lens):
        for j in range(pages[b]):
            blk = inp.block_table[b, j]
            n_valid = min(64, int(L) - 64 * j)
            assert np.isfinite(kf[blk, :n_valid]).all()
            assert np.isnan(kf[blk, n_valid:]).all()


def test_named_workloads_shapes():
    c = CONFIGS["gqa_causal_paged_f16_s2048"]
    assert c.flops_half_convention() == 2 * 128 * 2048 * 2048 * 32
    assert abs(c.flops_exact() / c.flops_half_convention() - 1) < 5e-4
    c3 = CONFIGS["chunked_prefill_bf16_512x4096"]
    assert c3.visible_pairs() == 4 * 1966336
    tiny = CONFIGS["tiny_causal_f16_d64"]
    assert tiny.flops_exact() == 2113536
