"""Every global address the kernels read or write stays inside its buffer (CPU only).

A model, in numpy, of the address arithmetic of the HIP kernels: the workgroup ->
(sequence, KV head, query block) mapping of the three prefill launch forms, their tile
ranges, the per-lane copy offsets (dma_off with the chunk swizzle), the page-id lookup
through the block table with out-of-range ids, the zero-chunk fallback for rows past a
key length, the Q fragment loads and the O / lse stores; for decode, the fixed-partition
split kernel and the balanced stream kernel with its plan (prefix sums, chunk, first
run of every range, cursor walk, partial slots). For each case every lane's 16-byte
source must lie inside its buffer (or be the zero chunk), every table read inside the
table, every store inside its output, and the 32-bit per-lane byte offsets must not
overflow. The composition of the 64-bit copy base from two wave-uniform halves is
checked for addresses whose low word has bit 31 set (the case a sign extension gets
wrong). The tail split's two launches and combine are modelled too (unit -> item and
key part, partial slots, row map). Nothing here runs on a GPU.
"""
import math

import numpy as np
import pytest

PAGE = 64
CUS = 256


# ------------------------------------------------------------------ shared helpers

def swz_prefill(D, row):
    # (the d = 256 narrow kernel XORs by 2 (row % 16) instead; any mask below the row's
    # chunk count only permutes the chunks of a row, so the sources checked are the same)
    row = np.asarray(row)
    if D == 64:
        k = (row >> 1) & 7
        return ((k & 1) << 2) | (k >> 1)
    r = row & 15
    return ((r & 3) << 2) | (r >> 2)


def swz_decode(D, row):
    row = np.asarray(row)
    if D == 64:
        k = (row >> 1) & 7
        return ((k & 3) << 1) | (k >> 2)
    r = row & 15
    return ((r & 7) << 1) | (r >> 3)


def readfirstlane(x):
    """__builtin_amdgcn_readfirstlane: a signed 32-bit int."""
    return np.array(x & 0xFFFFFFFF, dtype=np.uint64).astype(np.uint32).view(np.int32)


def compose_saddr(addr):
    """The 64-bit wave-uniform base of dma16_s, rebuilt from two readfirstlane halves
    widened through uint32 (as the kernel does)."""
    hi = np.uint64(readfirstlane(addr >> 32).view(np.uint32))
    lo = np.uint64(readfirstlane(addr).view(np.uint32))
    return int((hi << np.uint64(32)) | lo)


def tile_sources(D, swz, base, rs, row_ok):
    """Element offsets of the 16-byte sources of one 64-row K (or V) tile copy.

    The copy is NW * NIW wave instructions of 64 lanes; instruction i covers rows
    i*RPI .. i*RPI + RPI - 1, lane l row i*RPI + l // CPR and source chunk
    (l % CPR) ^ swz(row). Returns (offset [64*CPR], from_zero_chunk [64*CPR],
    dma_off bytes [64*CPR]) over all rows and lanes."""
    CPR = D // 8
    rows = np.repeat(np.arange(PAGE), CPR)
    pc = np.tile(np.arange(CPR), PAGE)
    dma_off = (rows * rs + ((pc ^ swz(D, rows)) << 3)) * 2
    off = base + dma_off // 2
    zero = ~row_ok[rows]
    return off, zero, dma_off


def assert_inside(off, zero, n_elems, what):
    live = off[~zero]
    assert live.size == 0 or (live.min() >= 0 and live.max() + 8 <= n_elems), \
        f"{what}: 16-byte source outside [0, {n_elems}) elements: {live.min()}..{live.max() + 8}"


# ------------------------------------------------------------------ prefill model

def prefill_form(D, causal, G, Sq, Sk, B, Hkv):
    """(NG, NW, PAIR, bq) chosen by the host for a launch (launch_one)."""
    if D == 128:
        diag_heavy = causal and G == 1 and Sk < 8192
        bq = 256 // G
        blocks8 = -(-Sq // bq) * Hkv * B
        if not diag_heavy and (2 * blocks8 >= 3 * CUS if causal else blocks8 >= CUS):
            return 1, 8, False, bq
    bq = 128 // G
    nq = -(-Sq // bq)
    blocks = nq * Hkv * B
    if D <= 128 and causal and blocks < 2048:
        if nq > 1 and blocks >= 2 * CUS:
            return 2, 4, True, bq
        return 2, 4, False, bq
    return 1, 4, False, bq


def check_prefill(D, B, Hq, Hkv, Sq, Sk, causal, paged, layout="bshd", lens=None, bad_ids=(),
                  cu=None):
    G = Hq // Hkv
    NG, NW, PAIR, bq = prefill_form(D, causal, G, Sq, Sk, B, Hkv)
    lens = np.full(B, Sk) if lens is None else np.asarray(lens)
    # strides (elements), as attn_api.cpp sets them
    if layout == "bshd":
        q_sb, q_sh, q_ss = Sq * Hq * D, D, Hq * D
        kv_sb, kv_sh, kv_ss = Sk * Hkv * D, D, Hkv * D
    else:
        q_sb, q_sh, q_ss = Hq * Sq * D, Sq * D, D
        kv_sb, kv_sh, kv_ss = Hkv * Sk * D, Sk * D, D
    if cu is not None:
        q_sb = 0
        total_q = int(cu[-1])
        q_elems = total_q * Hq * D
    else:
        q_elems = B * Sq * Hq * D
    pages_per_seq = -(-Sk // PAGE)
    if paged:
        num_blocks = B * pages_per_seq
        max_blocks = pages_per_seq
        table = np.random.default_rng(0).permutation(num_blocks).astype(np.int64).reshape(B, max_blocks)
        for (bb, jj, val) in bad_ids:
            table[bb, jj] = val
        kv_elems = num_blocks * PAGE * Hkv * D
        rs = Hkv * D
    else:
        kv_elems = B * Sk * Hkv * D
        rs = kv_ss
    assert max(rs * (PAGE - 1) * 2 + 2 * D, 0) < 2 ** 32, "dma_off overflows 32 bits"

    nq = -(-Sq // bq)
    nu = (nq + 1) // 2 if PAIR else nq
    grid = nu * Hkv * B
    rows_w = np.arange(NW * 32)                 # query rows of a group (wave * 32 + lq)
    visited = np.zeros((B, Hq, Sq), dtype=np.int64)
    for bx in range(grid):
        nx, xcd = grid, bx & 7
        per, extra = nx >> 3, nx & 7
        lid = xcd * per + min(xcd, extra) + (bx >> 3)
        unit, bh = lid % nu, lid // nu
        b, kvh = bh % B, bh // B
        assert 0 <= b < B and 0 <= kvh < Hkv
        L = min(max(int(lens[b]), 0), Sk)
        if cu is not None:
            c0 = int(cu[b])
            sq = min(max(int(cu[b + 1]) - c0, 0), Sq)
            qrow0 = c0
        else:
            sq, qrow0 = Sq, 0
        off = L - sq
        for it in range(2 if PAIR else 1):
            qblk = nq - 1 - unit if it == 0 else unit
            if it == 1 and qblk >= nq - 1 - unit:
                break
            q0 = qblk * bq
            hig = rows_w // bq
            rpos = q0 + (rows_w - hig * bq)
            rh = kvh * G + hig
            rok = (hig < G) & (rpos < sq)
            # Q fragments / O rows / lse of the rows this workgroup owns
            qi = b * q_sb + rh[rok] * q_sh + (qrow0 + rpos[rok]) * q_ss
            assert qi.size == 0 or (qi.min() >= 0 and qi.max() + D <= q_elems), "Q/O row outside the buffer"
            if cu is None:
                li = (b * Hq + rh[rok]) * Sq + rpos[rok]
                assert li.size == 0 or li.max() < B * Hq * Sq
                np.add.at(visited, (b, rh[rok], rpos[rok]), 1)
            else:
                li = rh[rok] * total_q + qrow0 + rpos[rok]
                assert li.size == 0 or li.max() < Hq * total_q
            # tile range and its split over the groups
            pmax = min(q0 + bq, sq) - 1
            kv_end = min(L, pmax + off + 1) if causal else L
            n_tiles = (kv_end + PAGE - 1) // PAGE if (kv_end > 0 and q0 < sq) else 0
            h = (n_tiles + NG - 1) // NG
            for grp in range(NG):
                j0, j1 = grp * h, min(n_tiles, grp * h + h)
                for j in range(j0, j1):
                    if paged:
                        ti = b * max_blocks + j
                        assert 0 <= ti < B * max_blocks, "block-table read outside the table"
                        pg = int(table.flat[ti])
                        page_ok = 0 <= pg < num_blocks
                        base = (pg if page_ok else 0) * PAGE * Hkv * D + kvh * D
                    else:
                        page_ok = True
                        base = b * kv_sb + kvh * kv_sh + j * PAGE * kv_ss
                    full = page_ok and (j + 1) * PAGE <= L
                    row_ok = np.full(PAGE, full) if full else \
                        np.array([page_ok and (j * PAGE + r < L) for r in range(PAGE)])
                    o, z, dma = tile_sources(D, swz_prefill, base, rs, row_ok)
                    assert dma.max() < 2 ** 32
                    assert_inside(o, z, kv_elems, f"prefill tile b={b} kvh={kvh} j={j}")
    if cu is None:
        # every query row of every head is owned by exactly one workgroup
        assert (visited == 1).all(), "a query row is written by no workgroup or by several"


PREFILL_CASES = [
    # (D, B, Hq, Hkv, Sq, Sk, causal, paged, layout, lens, bad_ids)
    (64, 2, 4, 2, 200, 200, True, True, "bshd", None, ()),               # the small d = 64 paged case
    (64, 2, 4, 2, 70, 190, True, True, "bshd", (190, 71), ()),
    (128, 2, 8, 2, 130, 300, True, True, "bshd", (300, 37), ((0, 2, -1), (1, 0, 10 ** 6))),
    (256, 1, 2, 1, 150, 150, True, True, "bshd", None, ()),
    (256, 2, 2, 2, 70, 133, False, False, "bshd", (133, 1), ()),
    (128, 2, 4, 4, 100, 257, False, False, "bhsd", None, ()),
    (64, 2, 4, 1, 129, 129, True, False, "bhsd", None, ()),
    (128, 1, 32, 8, 2048, 2048, True, True, "bshd", None, ()),           # paired two-group form
    (128, 1, 32, 8, 2080, 2080, True, True, "bshd", None, ((0, 5, -7),)),  # odd block count
    (128, 4, 16, 4, 512, 4096, True, True, "bshd", (4096, 4000, 3999, 1), ()),
    (64, 4, 64, 32, 1024, 1024, True, True, "bshd", None, ()),           # d = 64: four-wave blocks
    (128, 4, 64, 32, 1024, 1024, True, True, "bshd", None, ()),          # the same, eight-wave form
    (128, 2, 12, 4, 4100, 4100, True, True, "bshd", (4100, 3000), ((1, 3, 99999),)),
    (256, 1, 8, 8, 3000, 1000, False, False, "bshd", None, ()),
    # eight-wave launches with one (non-causal) or one and a half (causal) items per CU
    (128, 1, 16, 16, 4096, 4096, False, False, "bshd", None, ()),
    (128, 1, 32, 8, 3072, 3072, True, True, "bshd", None, ((0, 7, -3),)),
    (128, 2, 32, 8, 2048, 2048, True, True, "bshd", (2048, 1500), ()),
    (128, 1, 48, 16, 4096, 4096, True, True, "bshd", None, ()),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: f"d{c[0]}_B{c[1]}_{c[2]}x{c[3]}_{c[4]}x{c[5]}"
                         f"_{'causal' if c[6] else 'full'}_{'paged' if c[7] else 'dense'}_{c[8]}")
def test_prefill_addresses_in_bounds(case):
    D, B, Hq, Hkv, Sq, Sk, causal, paged, layout, lens, bad = case
    check_prefill(D, B, Hq, Hkv, Sq, Sk, causal, paged, layout, lens, bad)


def test_prefill_packed_query_addresses_in_bounds():
    cu = np.array([0, 100, 100, 357, 421])
    check_prefill(128, 4, 8, 2, 257, 1000, True, True, lens=(300, 50, 200, 1000), cu=cu)
    check_prefill(64, 3, 4, 4, 200, 130, False, False, lens=(130, 7, 130), cu=np.array([0, 33, 233, 234]))


def check_tail_split(D, B, Hq, Hkv, Sq, Sk, tail, parts, paged=False, lens=None, causal=False):
    """The tail split of a non-causal one-group launch (plan_one / launch_one and the
    split mode of both prefill kernels): the main launch takes items [0, N - tail), the
    split launch's unit u (through the same XCD permutation) takes part u % parts of item
    N - tail + u / parts; partial rows, partial slots and row-map entries stay inside the
    workspace the plan sizes; part 0 writes every row-map entry once; together the two
    launches own every query row exactly once; the combine reads only inside the
    partials."""
    G = Hq // Hkv
    NG, NW, PAIR, bq = prefill_form(D, causal, G, Sq, Sk, B, Hkv)
    if causal:
        # a causal launch splits only when it has few items, every one of them: in place
        # of a two-group launch (then in the one-group four-wave form), or at d = 256
        assert tail == -(-Sq // bq) * Hkv * B and not PAIR
        assert NG == 2 or D == 256
        NG, NW = 1, 4
    assert NG == 1 and not PAIR
    R = 16 * 8 if D == 256 else 32 * NW            # rows per item (narrow: 8 waves x 16)
    assert R == NW * 32                            # the same rows as the four-wave model
    lens = np.full(B, Sk) if lens is None else np.asarray(lens)
    nq = -(-Sq // bq)
    N = nq * Hkv * B
    assert 0 < tail <= N and 2 <= parts <= 64
    q_sb, q_sh, q_ss = Sq * Hq * D, D, Hq * D
    kv_sb, kv_sh, kv_ss = Sk * Hkv * D, D, Hkv * D
    pages_per_seq = -(-Sk // PAGE)
    if paged:
        num_blocks = B * pages_per_seq
        table = np.random.default_rng(1).permutation(num_blocks).reshape(B, pages_per_seq)
        kv_elems, rs = num_blocks * PAGE * Hkv * D, Hkv * D
    else:
        kv_elems, rs = B * Sk * Hkv * D, kv_ss
    o_elems = B * Sq * Hq * D
    rows = tail * R                                # workspace layout of the plan
    part_o_elems, part_lse_elems = rows * parts * D, rows * parts
    owned = np.zeros((B, Hq, Sq), dtype=np.int64)
    row_map = np.full(rows, -2, dtype=np.int64)    # -2: never written
    rows_w = np.arange(R)

    def item_rows(item):
        unit, bh = item % nq, item // nq
        b, kvh = bh % B, bh // B
        q0 = (nq - 1 - unit) * bq
        hig = rows_w // bq
        rpos = q0 + (rows_w - hig * bq)
        rh = kvh * G + hig
        rok = (hig < G) & (rpos < Sq)
        L = min(max(int(lens[b]), 0), Sk)
        pmax = min(q0 + bq, Sq) - 1
        kv_end = min(L, pmax + (L - Sq) + 1) if causal else L
        n_tiles = (kv_end + PAGE - 1) // PAGE if (kv_end > 0 and q0 < Sq) else 0
        return b, kvh, rh, rpos, rok, L, n_tiles

    def copy_tiles(b, kvh, L, j0, j1):
        for j in range(j0, j1):
            if paged:
                pg = int(table[b, j])
                base = pg * PAGE * Hkv * D + kvh * D
            else:
                base = b * kv_sb + kvh * kv_sh + j * PAGE * kv_ss
            full = (j + 1) * PAGE <= L
            row_ok = np.full(PAGE, full) if full else np.array([j * PAGE + r < L for r in range(PAGE)])
            o, z, dma = tile_sources(D, swz_prefill, base, rs, row_ok)
            assert dma.max() < 2 ** 32
            assert_inside(o, z, kv_elems, f"tail-split tile b={b} kvh={kvh} j={j}")

    def xcd_lid(bx, nx):
        per, extra, xcd = nx >> 3, nx & 7, bx & 7
        return xcd * per + min(xcd, extra) + (bx >> 3)

    # main launch: items [0, N - tail), whole key ranges, rows written to O directly
    n_main = N - tail
    lids = sorted(xcd_lid(bx, n_main) for bx in range(n_main))
    assert lids == list(range(n_main))
    for item in range(n_main):
        b, kvh, rh, rpos, rok, L, n_tiles = item_rows(item)
        np.add.at(owned, (b, rh[rok], rpos[rok]), 1)
    # split launch
    nx = tail * parts
    seen = set()
    for bx in range(nx):
        lid = xcd_lid(bx, nx)
        assert 0 <= lid < nx and lid not in seen
        seen.add(lid)
        item, part = n_main + lid // parts, lid % parts
        assert n_main <= item < N
        b, kvh, rh, rpos, rok, L, n_tiles = item_rows(item)
        tp = -(-n_tiles // parts) if n_tiles else 0
        j0 = min(part * tp, n_tiles)
        j1 = min(n_tiles, j0 + tp)
        assert 0 <= j0 <= j1 <= n_tiles
        copy_tiles(b, kvh, L, j0, j1)
        prow = (lid // parts) * R + rows_w
        assert prow.min() >= 0 and prow.max() < rows
        slot = prow * parts + part
        assert slot.max() < part_lse_elems and (slot.max() + 1) * D <= part_o_elems
        if part == 0:
            off = b * q_sb + rh * q_sh + rpos * q_ss
            assert (row_map[prow] == -2).all(), "a row-map entry written twice"
            row_map[prow] = np.where(rok, off, -1)
            assert off[rok].size == 0 or (off[rok].min() >= 0 and off[rok].max() + D <= o_elems)
            np.add.at(owned, (b, rh[rok], rpos[rok]), 1)
    assert (row_map != -2).all(), "a row-map entry never written"
    # combine: pair i reads slots i * parts + s, s < parts, and writes row_map[i] (if >= 0)
    pairs = np.arange(rows)
    assert ((pairs * parts + parts - 1) < part_lse_elems).all()
    assert ((pairs * parts + parts) * D <= part_o_elems).all()
    assert (owned == 1).all(), "a query row is owned by no launch or by several"


TAIL_CASES = [
    # (D, B, Hq, Hkv, Sq, Sk, tail, parts, paged, lens)
    (128, 1, 4, 4, 1024, 4096, 32, 8, False, None),          # every item split (first round)
    (128, 2, 8, 2, 300, 900, 20, 4, True, (900, 640)),       # the graph-test shape
    (64, 2, 8, 2, 200, 700, 8, 5, True, (700, 0)),           # a sequence with no key
    (128, 1, 16, 2, 90, 150, 1, 64, True, None),             # 64 parts of 3 tiles
    (256, 2, 4, 2, 130, 500, 6, 5, True, (500, 64)),         # narrow d = 256 form
    (128, 1, 17, 17, 16384, 256, 64, 4, False, None),        # eight-wave form, quarter-full round
    (256, 1, 5, 5, 8192, 512, 64, 4, False, None),           # narrow form, 320 items
]
CAUSAL_TAIL_CASES = [
    # causal launches with few items: every item split, four-wave one-group form
    (128, 2, 16, 4, 256, 4096, 64, 8, True, (4096, 3000)),   # chunked prefill, ragged keys
    (128, 2, 8, 2, 200, 700, 28, 3, True, (700, 300)),
    (64, 1, 4, 4, 300, 300, 12, 4, False, None),              # self-attention, empty parts
    (128, 2, 16, 4, 90, 60, 24, 2, True, (60, 0)),           # keys shorter than queries
    (256, 2, 4, 2, 150, 600, 12, 3, True, (600, 200)),       # narrow d = 256 form
    (256, 1, 16, 4, 512, 8192, 64, 4, False, None),
]


@pytest.mark.parametrize("case", TAIL_CASES, ids=lambda c: f"d{c[0]}_B{c[1]}_{c[2]}x{c[3]}_{c[4]}x{c[5]}_t{c[6]}p{c[7]}")
def test_tail_split_addresses_in_bounds(case):
    D, B, Hq, Hkv, Sq, Sk, tail, parts, paged, lens = case
    check_tail_split(D, B, Hq, Hkv, Sq, Sk, tail, parts, paged, lens)


@pytest.mark.parametrize("case", CAUSAL_TAIL_CASES, ids=lambda c: f"d{c[0]}_B{c[1]}_{c[2]}x{c[3]}_{c[4]}x{c[5]}_p{c[7]}")
def test_causal_split_addresses_in_bounds(case):
    D, B, Hq, Hkv, Sq, Sk, tail, parts, paged, lens = case
    check_tail_split(D, B, Hq, Hkv, Sq, Sk, tail, parts, paged, lens, causal=True)


def test_long_workload_launch_form_and_offsets():
    # the long non-causal bf16 workload runs the eight-wave form; its copy offsets fit 32 bits
    assert prefill_form(128, False, 1, 16384, 16384, 4, 16)[:2] == (1, 8)
    o, z, dma = tile_sources(128, swz_prefill, 0, 16 * 128, np.ones(PAGE, bool))
    assert dma.max() < 2 ** 32 and not z.any()


# ------------------------------------------------------------------ decode model

def decode_inputs(lens, Hkv, D, bad_ids=()):
    lens = np.asarray(lens)
    pages = [-(-int(L) // PAGE) for L in lens]
    num_blocks = max(1, sum(pages))
    max_blocks = max(1, max(pages))
    perm = np.random.default_rng(1).permutation(num_blocks)
    table = np.zeros((len(lens), max_blocks), dtype=np.int64)
    s = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[s:s + n]
        s += n
    for (bb, jj, val) in bad_ids:
        table[bb, jj] = val
    return table, num_blocks, max_blocks


def decode_page_copy(D, pg, num_blocks, Hkv, kvh, key0, end):
    rs = Hkv * D
    page_ok = 0 <= pg < num_blocks
    base = (pg if page_ok else 0) * PAGE * rs + kvh * D
    full = page_ok and key0 + PAGE <= end
    row_ok = np.full(PAGE, full) if full else np.array([page_ok and key0 + r < end for r in range(PAGE)])
    return tile_sources(D, swz_decode, base, rs, row_ok)


def check_decode_split(D, lens, Hq, Hkv, splits, bad_ids=()):
    """decode_split_kernel: one workgroup per (KV head, sequence, partition)."""
    B, G = len(lens), Hq // Hkv
    table, num_blocks, max_blocks = decode_inputs(lens, Hkv, D, bad_ids)
    max_seqlen_k = int(max(lens)) if len(lens) else 0
    part = -(-max_seqlen_k // splits)
    part = -(-part // PAGE) * PAGE or PAGE
    kv_elems = num_blocks * PAGE * Hkv * D
    NST = 512 // D
    written = np.zeros((B, Hq, splits), dtype=np.int64)
    for kvh in range(Hkv):
        for b in range(B):
            for split in range(splits):
                L = min(max(int(lens[b]), 0), max_seqlen_k)
                start = split * part
                end = min(start + part, L)
                out_row0 = (b * Hq + kvh * G) * splits + split
                rows = out_row0 + np.arange(G) * splits
                assert rows.max() < B * Hq * splits
                written[b, kvh * G:(kvh + 1) * G, split] += 1
                if start >= end:
                    continue
                first_page = start // PAGE
                n_pages = (end - start + PAGE - 1) // PAGE
                # page ids prefetched: indices < n_pages of the partition's table slice
                reads = list(range(min(NST - 1, n_pages))) + ([NST - 1] if NST - 1 < n_pages else []) + \
                    [i + NST for i in range(n_pages) if i + NST < n_pages]
                for k in reads:
                    ti = b * max_blocks + first_page + k
                    assert 0 <= ti < B * max_blocks, "block-table read outside the table"
                # Q: lane lr < G reads head kvh*G + lr
                assert (b * Hq + kvh * G + (G - 1)) * D + D <= B * Hq * D
                for k in range(n_pages):
                    pg = int(table.flat[b * max_blocks + first_page + k])
                    o, z, _ = decode_page_copy(D, pg, num_blocks, Hkv, kvh, start + k * PAGE, end)
                    assert_inside(o, z, kv_elems, f"decode split b={b} kvh={kvh} split={split} page={k}")
    assert (written == 1).all(), "a partition slot is written by no workgroup or by several"


def decode_plan(lens, max_seqlen_k, splits, nwk):
    """decode_plan_kernel: prefix[b], chunk, the first run of every range, total, ranges."""
    pages = [(min(max(int(L), 0), max_seqlen_k) + PAGE - 1) // PAGE for L in lens]
    prefix = np.concatenate([[0], np.cumsum(pages)]).astype(np.int64)
    total = int(prefix[-1])
    chunk = max((total + nwk - 1) // nwk, 1)
    rmax = (max_seqlen_k + PAGE - 1) // PAGE
    if splits > 1:
        chunk = max(chunk, (rmax + splits - 2) // (splits - 1))
    start = {}
    for b, r in enumerate(pages):
        u = int(prefix[b])
        j = (u + chunk - 1) // chunk
        while j * chunk < u + r:
            assert j < 1024, "plan writes past its start table"
            start[j] = b
            j += 1
    ranges = (total + chunk - 1) // chunk if total > 0 else 0
    assert ranges <= nwk
    return pages, prefix, total, chunk, start, ranges


def check_decode_stream(D, lens, Hq, Hkv, splits, bad_ids=()):
    """decode_stream_kernel: Hkv * nwk persistent workgroups walking the plan's ranges."""
    B, G = len(lens), Hq // Hkv
    table, num_blocks, max_blocks = decode_inputs(lens, Hkv, D, bad_ids)
    max_seqlen_k = int(max(lens))
    nwk = max(1, min(1024, CUS // Hkv))
    pages, prefix, total, chunk, start, ranges = decode_plan(lens, max_seqlen_k, splits, nwk)
    kv_elems = num_blocks * PAGE * Hkv * D
    slots = np.zeros((B, splits), dtype=np.int64)     # partial slots written (per KV head 0)
    for jr in range(nwk):
        if jr >= ranges:
            continue
        u_begin = jr * chunk
        n_units = min(chunk, total - u_begin)
        b = start[jr]
        c = {"b": b, "R": pages[b], "U": int(prefix[b]), "page": u_begin - int(prefix[b])}
        assert 0 <= c["page"] < c["R"]
        piece_u0 = u_begin
        for i in range(n_units):
            assert 0 <= c["b"] < B
            L = min(max(int(lens[c["b"]]), 0), max_seqlen_k)
            ti = c["b"] * max_blocks + c["page"]
            assert 0 <= ti < B * max_blocks, "block-table read outside the table"
            pg = int(table.flat[ti])
            for kvh in (0, Hkv - 1):
                o, z, _ = decode_page_copy(D, pg, num_blocks, Hkv, kvh, c["page"] * PAGE, L)
                assert_inside(o, z, kv_elems, f"decode stream run={c['b']} page={c['page']}")
            # Q block rows < G of sequence b
            assert (c["b"] * Hq + (Hkv - 1) * G + G - 1) * D + D <= B * Hq * D
            run_end = c["page"] == c["R"] - 1
            if run_end or i == n_units - 1:
                slot = piece_u0 // chunk - c["U"] // chunk
                assert 0 <= slot < splits, f"partial slot {slot} outside [0, {splits})"
                slots[c["b"], slot] += 1
                piece_u0 = u_begin + i + 1
            if i + 1 < n_units:
                c["page"] += 1
                if c["page"] == c["R"]:
                    c["U"] += c["R"]
                    c["page"] = 0
                    while True:
                        c["b"] += 1
                        assert c["b"] < B, "cursor walked past the last sequence"
                        c["R"] = pages[c["b"]]
                        if c["R"] != 0:
                            break
    # every non-empty sequence's partitions cover its pages, one slot each, from slot 0 up
    for b in range(B):
        n = int((slots[b] > 0).sum())
        assert (slots[b] <= 1).all()
        if pages[b]:
            assert n >= 1 and (slots[b, :n] == 1).all()


DECODE_CASES = [
    # (D, lens, Hq, Hkv, splits, bad_ids)
    (128, (1, 63, 64, 65, 1000), 8, 2, 3, ()),
    (64, (333, 64, 2000), 16, 2, 16, ((2, 5, -1),)),
    (256, (900, 1, 190), 4, 2, 5, ((0, 1, 10 ** 7),)),
    (128, (0, 300, 0, 5000, 64), 8, 2, 16, ()),
    (128, tuple(int(x) for x in np.random.default_rng(4).integers(1024, 65537, size=32)), 32, 8, 16, ()),
    (64, tuple(int(x) for x in np.random.default_rng(5).integers(0, 700, size=48)), 8, 8, 2, ()),
    (128, (262144, 131071), 8, 2, 16, ()),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"d{c[0]}_B{len(c[1])}_s{c[4]}")
def test_decode_split_addresses_in_bounds(case):
    D, lens, Hq, Hkv, splits, bad = case
    if sum(lens) > 500000:
        pytest.skip("the fixed-partition model walks every page; covered by the stream model")
    check_decode_split(D, lens, Hq, Hkv, 1, bad)
    check_decode_split(D, lens, Hq, Hkv, splits, bad)


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"d{c[0]}_B{len(c[1])}_s{c[4]}")
def test_decode_stream_addresses_in_bounds(case):
    D, lens, Hq, Hkv, splits, bad = case
    if splits < 2:
        pytest.skip("the balanced kernel serves num_splits >= 2")
    check_decode_stream(D, lens, Hq, Hkv, splits, bad)


def test_copy_base_survives_bit31_of_the_low_word():
    # dma16_s rebuilds the 64-bit base from two readfirstlane results; a low word with
    # bit 31 set must not be sign-extended into the high word
    for addr in (0x7F12_8000_0000, 0x7F12_FFFF_FFF0, 0x1_0000_0000, 0x7F12_7FFF_FFF0, 0x8000_0000):
        assert compose_saddr(addr) == addr
    # the unwidened composition (what the check guards against) would differ
    lo = int(readfirstlane(0x7F12_8000_0000))
    assert lo < 0 and ((0x7F12 << 32) | (lo & 0xFFFF_FFFF_FFFF_FFFF)) != 0x7F12_8000_0000


def test_random_sweep_addresses_in_bounds():
    """Every shape of the seeded random parity sweep (tests/test_random_shapes_gpu.py)
    through the same address models, before any of it runs on a device: the prefill
    launch form the host picks (and, for a forced split of a launch that qualifies, the
    split units with every item in the tail), packed queries, and both decode kernels."""
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from test_random_shapes_gpu import N_DECODE, N_PACKED, N_PREFILL, draw_decode, draw_packed, draw_prefill
    for i in range(N_PREFILL):
        c, splits = draw_prefill(i)
        D, B, Hq, Hkv, Sq, Sk = c.head_dim, c.batch, c.heads_q, c.heads_kv, c.seqlen_q, c.seqlen_k
        paged = c.kv == "paged"
        check_prefill(D, B, Hq, Hkv, Sq, Sk, c.causal, paged, c.layout, c.seqlens_k)
        if splits < 2 or c.precise or c.layout != "bshd":
            continue
        NG, NW, PAIR, bq = prefill_form(D, c.causal, Hq // Hkv, Sq, Sk, B, Hkv)
        items = -(-Sq // bq) * Hkv * B
        few = 2 * items <= CUS and (NG == 2 or D == 256) and not PAIR
        if not c.causal or few:
            check_tail_split(D, B, Hq, Hkv, Sq, Sk, items, splits, paged, c.seqlens_k, causal=c.causal)
    for i in range(N_PACKED):
        c, q_lens = draw_packed(i)
        cu = np.concatenate([[0], np.cumsum(q_lens)])
        check_prefill(c.head_dim, c.batch, c.heads_q, c.heads_kv, c.seqlen_q, c.seqlen_k, c.causal,
                      c.kv == "paged", lens=c.seqlens_k, cu=cu)
    for i in range(N_DECODE):
        c, splits = draw_decode(i)
        check_decode_split(c.head_dim, c.lengths_fixed, c.heads_q, c.heads_kv, 1)
        if splits >= 2:
            check_decode_stream(c.head_dim, c.lengths_fixed, c.heads_q, c.heads_kv, splits)
