"""Pins for the fp64 oracle: closed forms, invariants, a library special case,
hand-derived golden fixtures, and planted mistakes that the pins must catch.

All CPU. Every check is written as a ``check_*`` helper so the mutation tests
at the bottom can run the same check against a deliberately broken oracle.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import materialised as oatt
from oracle import combine as ocomb
from oracle.brute import brute_row
from oracle.online import online_attention_rows

TOL = 1e-12


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _dense_case(seed, B=2, Sq=5, Sk=9, Hq=4, Hkv=2, d=8, layout="bshd"):
    q = rnd((B, Sq, Hq, d), seed)
    k = rnd((B, Sk, Hkv, d), seed + 1)
    v = rnd((B, Sk, Hkv, d), seed + 2)
    if layout == "bhsd":
        q, k, v = (x.transpose(0, 2, 1, 3).copy() for x in (q, k, v))
    return q, k, v


# ----------------------------------------------------------------------------- checks

def check_weights_are_a_distribution(seed=0):
    for causal in (False, True):
        for Sq, Sk in ((1, 1), (3, 3), (4, 11), (7, 64)):
            qr = rnd((Sq, 16), seed)
            K = rnd((Sk, 16), seed + 1)
            V = rnd((Sk, 16), seed + 2)
            _, _, a = oatt.attention_rows(qr, K, V, np.arange(Sq), Sk, Sq, causal, 0.25,
                                          return_weights=True)
            assert (a >= 0).all()
            np.testing.assert_allclose(a.sum(axis=1), 1.0, atol=TOL, rtol=0)
            if causal:
                i = np.arange(Sq)[:, None]
                j = np.arange(Sk)[None, :]
                assert (a[j > i + Sk - Sq] == 0).all()
                # visible count of row i is S_k - S_q + i + 1
                np.testing.assert_array_equal((a > 0).sum(axis=1), Sk - Sq + np.arange(Sq) + 1)


def check_convex_hull(seed=1):
    q, k, v = _dense_case(seed, Sq=6, Sk=6)
    for causal in (False, True):
        O, _ = oracle.attention(q, k, v, causal=causal)
        G = q.shape[2] // k.shape[2]
        for b in range(q.shape[0]):
            for h in range(q.shape[2]):
                for i in range(q.shape[1]):
                    nvis = i + 1 if causal else k.shape[1]
                    rows = v[b, :nvis, h // G]
                    assert (O[b, i, h] >= rows.min(axis=0) - TOL).all()
                    assert (O[b, i, h] <= rows.max(axis=0) + TOL).all()


def check_uniform_scores_give_mean(seed=2):
    B, Sq, Sk, Hq, Hkv, d = 2, 5, 12, 4, 2, 8
    q = np.zeros((B, Sq, Hq, d))
    k = rnd((B, Sk, Hkv, d), seed)
    v = rnd((B, Sk, Hkv, d), seed + 1)
    for causal in (False, True):
        O, lse = oracle.attention(q, k, v, causal=causal)
        csum = np.cumsum(v, axis=1)
        for i in range(Sq):
            n = (Sk - Sq + i + 1) if causal else Sk
            mean = csum[:, n - 1] / n                    # [B, Hkv, d]
            want = np.repeat(mean, Hq // Hkv, axis=1)    # head h -> kv head h // G
            np.testing.assert_allclose(O[:, i], want, atol=TOL, rtol=0)
            np.testing.assert_allclose(lse[:, :, i], math.log(n), atol=TOL, rtol=0)


def check_single_key():
    q, k, v = _dense_case(3, Sq=4, Sk=1)
    O, _ = oracle.attention(q, k, v, causal=False)
    np.testing.assert_allclose(O, np.repeat(v, 2, axis=2).repeat(4, axis=1), atol=TOL, rtol=0)
    # causal with S_q = S_k = 1
    O1, _ = oracle.attention(q[:, :1], k, v, causal=True)
    np.testing.assert_allclose(O1[:, 0], np.repeat(v[:, 0], 2, axis=1), atol=TOL, rtol=0)


def check_dominant_score():
    d, Sk = 16, 10
    qr = rnd((1, d), 4)
    K = rnd((Sk, d), 5)
    V = rnd((Sk, d), 6)
    jstar = 6
    K[jstar] = 50.0 * qr[0]           # score gap far above 40 in natural-log units
    O, _ = oatt.attention_rows(qr, K, V, np.array([0]), Sk, 1, False, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(O[0], V[jstar], atol=TOL, rtol=0)
    # the same with very large raw scores: needs the max subtraction to stay finite
    K2 = K.copy()
    K2[jstar] = 400.0 * qr[0]
    O2, lse2 = oatt.attention_rows(qr, K2, V, np.array([0]), Sk, 1, False, 1.0)
    assert np.isfinite(O2).all() and np.isfinite(lse2).all()
    np.testing.assert_allclose(O2[0], V[jstar], atol=TOL, rtol=0)


def check_masked_keys_ignored(seed=7):
    B, Sq, Sk, H, d = 1, 4, 9, 1, 8
    q = rnd((B, Sq, H, d), seed)
    k = rnd((B, Sk, H, d), seed + 1)
    v = rnd((B, Sk, H, d), seed + 2)
    O, _ = oracle.attention(q, k, v, causal=True)
    off = Sk - Sq
    for i in range(Sq):
        k2, v2 = k.copy(), v.copy()
        k2[:, i + off + 1:] = 1e6
        v2[:, i + off + 1:] = -1e6
        O2, _ = oracle.attention(q, k2, v2, causal=True)
        np.testing.assert_array_equal(O2[:, i], O[:, i])


def check_online_matches_materialised(seed=8):
    cases = [
        dict(B=1, Sq=9, Sk=9, Hq=2, Hkv=1, d=8, causal=True),
        dict(B=2, Sq=3, Sk=11, Hq=4, Hkv=2, d=8, causal=True),
        dict(B=1, Sq=4, Sk=7, Hq=2, Hkv=2, d=4, causal=False),
    ]
    for c in cases:
        q, k, v = _dense_case(seed, B=c["B"], Sq=c["Sq"], Sk=c["Sk"], Hq=c["Hq"], Hkv=c["Hkv"], d=c["d"])
        q = q * 3.0                                     # spread the scores
        O, lse = oracle.attention(q, k, v, causal=c["causal"])
        for T in (1, 2, 3, 7, 64, 128, c["Sk"]):
            for b in range(c["B"]):
                for h in range(c["Hq"]):
                    Oo, lo = online_attention_rows(q, k, v, b=b, h=h, rows=range(c["Sq"]),
                                                   causal=c["causal"], tile=T)
                    np.testing.assert_allclose(Oo, O[b, :, h], atol=TOL, rtol=0)
                    np.testing.assert_allclose(lo, lse[b, h], atol=TOL, rtol=0)


def check_online_matches_paged(seed=9):
    Sk, page, d = 150, 64, 8
    kl = rnd((1, Sk, 1, d), seed)
    vl = rnd((1, Sk, 1, d), seed + 1)
    q = rnd((1, 2, 1, d), seed + 2)
    table = np.array([[2, 0, 1]])
    kc = np.full((3, page, 1, d), np.nan)
    vc = np.full((3, page, 1, d), np.nan)
    for j in range(Sk):
        kc[table[0, j // page], j % page] = kl[0, j]
        vc[table[0, j // page], j % page] = vl[0, j]
    O, _ = oracle.attention(q, kc, vc, causal=True, block_table=table, seqlens_k=[Sk])
    Oo, _ = online_attention_rows(q, kc, vc, b=0, h=0, rows=[0, 1], causal=True, tile=64,
                                  block_table=table, seqlens_k=[Sk])
    np.testing.assert_allclose(Oo, O[0, :, 0], atol=TOL, rtol=0)


def check_two_key_closed_form(seed=10):
    d = 8
    qr = rnd((1, d), seed)
    K = rnd((2, d), seed + 1)
    V = rnd((2, d), seed + 2)
    tau = 1.0 / math.sqrt(d)
    s0 = tau * sum(qr[0, c] * K[0, c] for c in range(d))
    s1 = tau * sum(qr[0, c] * K[1, c] for c in range(d))
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))     # noqa: E731
    want = sig(s0 - s1) * V[0] + sig(s1 - s0) * V[1]
    q = qr.reshape(1, 1, 1, d)
    O, _ = oracle.attention(q, K.reshape(1, 2, 1, d), V.reshape(1, 2, 1, d), causal=False)
    np.testing.assert_allclose(O[0, 0, 0], want, atol=TOL, rtol=0)


def _torch_ref(q, k, v, causal):
    """torch CPU SDPA in float64 with an explicit bottom-right boolean mask (bshd in/out)."""
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3)
    G = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(G, dim=1)
    vt = vt.repeat_interleave(G, dim=1)
    Sq, Sk = qt.shape[2], kt.shape[2]
    mask = None
    if causal:
        mask = torch.ones(Sq, Sk, dtype=torch.bool).tril(diagonal=Sk - Sq)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    return out.permute(0, 2, 1, 3).numpy()


def check_torch_sdpa_special_case(seed=11):
    for (Sq, Sk, causal) in ((6, 6, True), (3, 10, True), (5, 8, False), (1, 7, False)):
        q, k, v = _dense_case(seed, B=2, Sq=Sq, Sk=Sk, Hq=4, Hkv=2, d=16)
        O, _ = oracle.attention(q, k, v, causal=causal)
        np.testing.assert_allclose(O, _torch_ref(q, k, v, causal), atol=TOL, rtol=0)
    # square causal equals torch's own (top-left) is_causal, since the two alignments agree
    q, k, v = _dense_case(seed, B=1, Sq=7, Sk=7, Hq=2, Hkv=2, d=16)
    O, _ = oracle.attention(q, k, v, causal=True)
    t = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v)), is_causal=True)
    np.testing.assert_allclose(O, t.permute(0, 2, 1, 3).numpy(), atol=TOL, rtol=0)


def check_affine_equivariance(seed=12):
    q, k, v = _dense_case(seed)
    for causal in (False, True):
        O, _ = oracle.attention(q, k, v, causal=causal)
        O2, _ = oracle.attention(q, k, -2.5 * v + 0.75, causal=causal)
        np.testing.assert_allclose(O2, -2.5 * O + 0.75, atol=1e-11, rtol=0)


def check_key_permutation(seed=13):
    q, k, v = _dense_case(seed)
    perm = np.random.default_rng(seed).permutation(k.shape[1])
    O, _ = oracle.attention(q, k, v, causal=False)
    O2, _ = oracle.attention(q, k[:, perm], v[:, perm], causal=False)
    np.testing.assert_allclose(O2, O, atol=TOL, rtol=0)


def check_paged_equals_dense(seed=14):
    B, Sk, Hkv, d, page = 2, 130, 2, 8, 64
    q, k, v = _dense_case(seed, B=B, Sq=4, Sk=Sk, Hq=4, Hkv=Hkv, d=d)
    lens = np.array([130, 77])
    npages = -(-Sk // page)
    table = np.random.default_rng(seed).permutation(B * npages).reshape(B, npages)
    kc = np.full((B * npages, page, Hkv, d), np.nan)
    vc = np.full((B * npages, page, Hkv, d), np.nan)
    for b in range(B):
        for j in range(lens[b]):
            kc[table[b, j // page], j % page] = k[b, j]
            vc[table[b, j // page], j % page] = v[b, j]
    for causal in (False, True):
        Op, lp = oracle.attention(q, kc, vc, causal=causal, block_table=table, seqlens_k=lens)
        Od, ld = oracle.attention(q, k, v, causal=causal, seqlens_k=lens)
        np.testing.assert_array_equal(Op, Od)
        np.testing.assert_array_equal(lp, ld)


def check_gqa_equals_repeated_mha(seed=15):
    q, k, v = _dense_case(seed, Hq=8, Hkv=2)
    for causal in (False, True):
        O, _ = oracle.attention(q, k, v, causal=causal)
        O2, _ = oracle.attention(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), causal=causal)
        np.testing.assert_array_equal(O, O2)


def check_layouts_agree(seed=16):
    q, k, v = _dense_case(seed)
    for causal in (False, True):
        O, l = oracle.attention(q, k, v, causal=causal, layout="bshd")
        qb, kb, vb = (x.transpose(0, 2, 1, 3).copy() for x in (q, k, v))
        O2, l2 = oracle.attention(qb, kb, vb, causal=causal, layout="bhsd")
        np.testing.assert_array_equal(O2.transpose(0, 2, 1, 3), O)
        np.testing.assert_array_equal(l2, l)


def check_split_combine(seed=17):
    rng = np.random.default_rng(seed)
    q, k, v = _dense_case(seed, B=2, Sq=1, Sk=200, Hq=4, Hkv=2, d=8)
    q = 2.0 * q
    O, lse = oracle.attention(q, k, v, causal=False)
    random_edges = sorted(set(rng.choice(np.arange(1, 200), size=5, replace=False).tolist()))
    for inner in ([], [64, 128], [5, 6], random_edges):
        edges = [0, *inner, 200]
        bounds = list(zip(edges[:-1], edges[1:])) + [(200, 256)]      # the last split is empty
        po, pl = ocomb.split_partials(q, k, v, bounds=bounds)
        assert np.isneginf(pl[..., -1]).all()
        assert (po[..., -1, :] == 0).all()
        Oc, lc = ocomb.lse_combine(po, pl)
        np.testing.assert_allclose(Oc, O.transpose(0, 2, 1, 3), atol=TOL, rtol=0)
        np.testing.assert_allclose(lc, lse, atol=TOL, rtol=0)
    # an all-empty set of partials gives 0 / -inf
    Oe, le = ocomb.lse_combine(np.zeros((3, 4)), np.full(3, -np.inf))
    assert (Oe == 0).all() and np.isneginf(le)


def check_decode_causal_is_noncausal(seed=18):
    q, k, v = _dense_case(seed, Sq=1, Sk=37)
    O1, _ = oracle.attention(q, k, v, causal=True)
    O2, _ = oracle.attention(q, k, v, causal=False)
    np.testing.assert_array_equal(O1, O2)


def check_brute_force(seed=19):
    q, k, v = _dense_case(seed, B=1, Sq=3, Sk=6, Hq=2, Hkv=1, d=4)
    for causal in (False, True):
        O, _ = oracle.attention(q, k, v, causal=causal)
        for h in range(2):
            for i in range(3):
                nvis = (6 - 3 + i + 1) if causal else 6
                want = brute_row(list(q[0, i, h]), [list(r) for r in k[0, :nvis, 0]],
                                 [list(r) for r in v[0, :nvis, 0]], 0.5)
                np.testing.assert_allclose(O[0, i, h], want, atol=TOL, rtol=0)


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def check_golden_uniform_chunked(golden_dir):
    g = _load(golden_dir, "uniform_chunked_causal.json")
    d = g["head_dim"]
    q = np.array(g["q"]).reshape(1, -1, 1, d)
    k = np.array(g["k"]).reshape(1, -1, 1, d)
    v = np.array(g["v"]).reshape(1, -1, 1, d)
    O, _ = oracle.attention(q, k, v, causal=True)
    np.testing.assert_allclose(O[0, :, 0], g["expected_causal"], atol=g["tolerance"], rtol=0)
    O, _ = oracle.attention(q, k, v, causal=False)
    np.testing.assert_allclose(O[0, :, 0], g["expected_noncausal"], atol=g["tolerance"], rtol=0)


def check_golden_two_key(golden_dir):
    g = _load(golden_dir, "two_key_ln3.json")
    d = g["head_dim"]
    q = np.array(g["q"]).reshape(1, -1, 1, d)
    k = np.array(g["k"]).reshape(1, -1, 1, d)
    v = np.array(g["v"]).reshape(1, -1, 1, d)
    O, lse = oracle.attention(q, k, v, causal=False)
    np.testing.assert_allclose(O[0, :, 0], g["expected_noncausal"], atol=g["tolerance"], rtol=0)
    np.testing.assert_allclose(lse[0, 0], g["expected_lse"], atol=g["tolerance"], rtol=0)


def check_golden_gqa(golden_dir):
    g = _load(golden_dir, "gqa_head_map.json")
    vk = np.array(g["v_by_kv_head"])                # [Hkv, S_k, 1]
    v = vk.transpose(1, 0, 2)[None]                  # [1, S_k, Hkv, 1]
    k = np.zeros_like(v)
    q = np.zeros((1, 1, 4, 1))
    O, _ = oracle.attention(q, k, v, causal=False)
    np.testing.assert_allclose(O[0, 0, :, 0], g["expected_by_q_head"], atol=g["tolerance"], rtol=0)


def check_golden_paged(golden_dir):
    g = _load(golden_dir, "paged_gather.json")
    L, table = g["seqlen_k"], np.array([g["table"]])
    kc = np.zeros((2, 64, 1, 1))
    vc = np.full((2, 64, 1, 1), g["filler"])
    for j in range(L):
        vc[table[0, j // 64], j % 64, 0, 0] = j
    q = np.zeros((1, 1, 1, 1))
    O, _ = oracle.attention(q, kc, vc, causal=False, block_table=table, seqlens_k=[L])
    np.testing.assert_allclose(O[0, 0, 0, 0], g["expected"], atol=g["tolerance"], rtol=0)


CHECKS = [
    check_weights_are_a_distribution, check_convex_hull, check_uniform_scores_give_mean,
    check_single_key, check_dominant_score, check_masked_keys_ignored,
    check_online_matches_materialised, check_online_matches_paged, check_two_key_closed_form,
    check_torch_sdpa_special_case, check_affine_equivariance, check_key_permutation,
    check_paged_equals_dense, check_gqa_equals_repeated_mha, check_layouts_agree,
    check_split_combine, check_decode_causal_is_noncausal, check_brute_force,
]
GOLDEN = [check_golden_uniform_chunked, check_golden_two_key, check_golden_gqa, check_golden_paged]


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__[6:])
def test_oracle_pin(check):
    check()


@pytest.mark.parametrize("check", GOLDEN, ids=lambda f: f.__name__[6:])
def test_oracle_golden(check, golden_dir):
    check(golden_dir)


# ----------------------------------------------------------------------------- planted mistakes

def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_plant_top_left_mask(monkeypatch, golden_dir):
    def top_left(i, j, L, S_q, causal):
        vis = j < L
        return vis & (j <= i) if causal else vis
    monkeypatch.setattr(oatt, "is_visible", top_left)
    assert _fails(check_golden_uniform_chunked, golden_dir)
    assert _fails(check_torch_sdpa_special_case)
    assert _fails(check_online_matches_materialised)


def test_plant_wrong_head_map(monkeypatch, golden_dir):
    monkeypatch.setattr(oatt, "kv_head_of", lambda h, G: h % G)
    assert _fails(check_golden_gqa, golden_dir)
    assert _fails(check_torch_sdpa_special_case)
    assert _fails(check_uniform_scores_give_mean)


def test_plant_wrong_scale(monkeypatch, golden_dir):
    real = oatt.attention_rows

    def scaled(q_rows, K, V, rows, L, S_q, causal, scale, **kw):
        return real(q_rows, K, V, rows, L, S_q, causal, scale * scale, **kw)   # 1/d instead of 1/sqrt(d)
    monkeypatch.setattr(oatt, "attention_rows", scaled)
    assert _fails(check_golden_two_key, golden_dir)
    assert _fails(check_two_key_closed_form)
    assert _fails(check_torch_sdpa_special_case)


def test_plant_gather_ignores_table(monkeypatch, golden_dir):
    def physical(cache, table_row, L, kvh):
        page = cache.shape[1]
        j = np.arange(L)
        return cache[j // page, j % page, kvh, :]
    monkeypatch.setattr(oatt, "gather_kv", physical)
    assert _fails(check_golden_paged, golden_dir)
    assert _fails(check_paged_equals_dense)


def test_plant_transposed_v(monkeypatch):
    real = oatt.attention_rows

    def swapped(q_rows, K, V, rows, L, S_q, causal, scale, **kw):
        return real(q_rows, V, K, rows, L, S_q, causal, scale, **kw)          # K and V exchanged
    monkeypatch.setattr(oatt, "attention_rows", swapped)
    assert _fails(check_torch_sdpa_special_case)
    assert _fails(check_affine_equivariance)


def test_plant_no_max_subtraction(monkeypatch):
    def no_max(q_rows, K, V, rows, L, S_q, causal, scale, key_range=None, return_weights=False):
        s = scale * (q_rows @ K.T)
        j = np.arange(K.shape[0])
        vis = oatt.is_visible(np.asarray(rows)[:, None], j[None, :], L, S_q, causal)
        with np.errstate(over="ignore", invalid="ignore"):
            w = np.where(vis, np.exp(s), 0.0)
            a = w / w.sum(axis=1, keepdims=True)
            return a @ V, np.log(w.sum(axis=1))
    monkeypatch.setattr(oatt, "attention_rows", no_max)
    assert _fails(check_dominant_score)


def test_plant_combine_without_weights(monkeypatch):
    def plain_mean(partial_o, partial_lse):
        ok = np.isfinite(partial_lse)
        O = (partial_o * ok[..., None]).sum(axis=-2) / ok.sum(axis=-1)[..., None]
        return O, partial_lse.max(axis=-1)
    monkeypatch.setattr(ocomb, "lse_combine", plain_mean)
    assert _fails(check_split_combine)


# ---------------------------------------------------------------- bfloat16 output rounding
# The benchmark page measures bf16 outputs in three rounding modes: to nearest with ties
# to even (RTNE), to nearest with ties away from zero (RTNA), toward zero (RTZ). Pins:
# hand-derived values, the library's own RTNE conversion (torch float32 -> bfloat16),
# and bit-level formulations on float32 patterns that share nothing with the oracle's
# exact arithmetic.

from oracle.rounding import round_bf16, round_bf16_scalar  # noqa: E402

# (x, RTNE, RTNA, RTZ); bfloat16 keeps 7 fraction bits: next value after 1 is 1 + 2^-7.
ROUND_CASES = [
    (1.0, 1.0, 1.0, 1.0),
    (1 + 2 ** -8, 1.0, 1 + 2 ** -7, 1.0),                      # exact tie, even neighbour is 1
    (1 + 3 * 2 ** -8, 1 + 2 * 2 ** -7, 1 + 2 * 2 ** -7, 1 + 2 ** -7),   # tie, even neighbour is above
    (-(1 + 2 ** -8), -1.0, -(1 + 2 ** -7), -1.0),              # sign-symmetric
    (1 + 2 ** -9, 1.0, 1.0, 1.0),                              # below the tie
    (1 + 2 ** -8 + 2 ** -20, 1 + 2 ** -7, 1 + 2 ** -7, 1.0),  # just above the tie
    (3.4e38, math.inf, math.inf, (2 - 2 ** -7) * 2 ** 127),    # overflow: RTZ stays finite
    (-(2 ** -134), -0.0, -(2 ** -133), -0.0),                  # half the smallest subnormal
    (2.5 * 2 ** -133, 2 * 2 ** -133, 3 * 2 ** -133, 2 * 2 ** -133),   # subnormal tie
]


@pytest.mark.parametrize("x,rtne,rtna,rtz", ROUND_CASES)
def test_round_bf16_hand_values(x, rtne, rtna, rtz):
    for mode, want in (("rtne", rtne), ("rtna", rtna), ("rtz", rtz)):
        got = round_bf16_scalar(x, mode)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (x, mode, got, want)


def _random_f32(n, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n))).astype(np.float32)
    x[::7] = (x[::7].view(np.uint32) & 0xFFFF0000 | (1 << 15)).view(np.float32)   # exact ties
    return x


def test_round_bf16_rtne_matches_torch():
    x = _random_f32(4000, 1)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_bf16(x.astype(np.float64), "rtne"), want)


def test_round_bf16_bit_formulations():
    x = _random_f32(4000, 2)
    bits = x.view(np.uint32).astype(np.uint64)
    sign = bits & 0x80000000
    mag = bits & 0x7FFFFFFF
    rtz = (sign | (mag & 0x7FFF0000)).astype(np.uint32).view(np.float32).astype(np.float64)
    rtna = (sign | ((mag + 0x8000) & 0x7FFF0000)).astype(np.uint32).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(round_bf16(x.astype(np.float64), "rtz"), rtz)
    np.testing.assert_array_equal(round_bf16(x.astype(np.float64), "rtna"), rtna)


def test_round_bf16_properties():
    x = _random_f32(2000, 3).astype(np.float64)
    for mode in ("rtne", "rtna", "rtz"):
        r = round_bf16(x, mode)
        assert (r.astype(np.float32).view(np.uint32) & 0xFFFF).max() == 0     # on the bf16 grid
        ulp = np.exp2(np.floor(np.log2(np.abs(x))) - 7)
        if mode == "rtz":
            assert (np.abs(r) <= np.abs(x)).all() and (np.abs(x) - np.abs(r) < ulp).all()
        else:
            assert (np.abs(r - x) <= ulp / 2).all()


def test_round_bf16_keeps_shape_and_order():
    # a transposed (non-contiguous) view, as attention outputs in BSHD are
    x = _random_f32(2 * 3 * 5, 4).astype(np.float64).reshape(2, 3, 5).transpose(0, 2, 1)
    r = round_bf16(x, "rtz")
    assert r.shape == x.shape
    for idx in np.ndindex(*x.shape):
        assert r[idx] == round_bf16_scalar(float(x[idx]), "rtz")
