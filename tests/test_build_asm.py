"""The m0 invariant of the inline-asm LDS copies and the register budgets of the hot
kernels, checked on freshly compiled gfx950 assembly (CPU only: hipcc cross-compiles),
and the checkers themselves on small samples."""
import re

import pytest

from attention_forward_tiled_amd import build


def test_checker_accepts_the_copy_idiom_and_flags_other_uses():
    good = "\ts_mov_b32 m0, s39\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v[12:13], off\n\ts_endpgm\n"
    assert build.check_m0(good) == []
    assert build.check_m0("\ts_mov_b32 m0, s3\n\tv_add_f32 v1, v2, v3\n") != []       # no copy follows
    assert build.check_m0("\ts_mov_b32 s4, m0\n") != []                               # m0 read
    assert build.check_m0("\tv_movrels_b32 v1, v2\n") != []                           # implicit use
    assert build.check_m0("\ts_set_gpr_idx_on s2, gpr_idx(SRC0)\n") != []
    assert build.check_m0("\tv_mov_b32 v0, v1 ; comment naming m0\n") == []           # comments ignored


@pytest.fixture(scope="module")
def built(tmp_path_factory):
    # compile_all raises if any source's gfx950 assembly uses m0 outside the idiom
    d = str(tmp_path_factory.mktemp("asm"))
    build.compile_all(d, jobs=3)
    return d


def test_compiled_kernels_keep_m0_for_the_copies(built):
    asm = build.device_asm("prefill.hip", built)
    assert asm.count("global_load_lds_dwordx4") > 0
    assert build.check_m0(asm) == []


def test_resource_parser_reads_the_metadata_block():
    asm = ("\t.text\namdhsa.kernels:\n  - .agpr_count:     4\n    .args:\n      - .offset:         0\n"
           "    .group_segment_fixed_size: 1024\n    .name:           k1\n    .private_segment_fixed_size: 8\n"
           "    .sgpr_count:     20\n    .sgpr_spill_count: 0\n    .vgpr_count:     40\n    .vgpr_spill_count: 2\n"
           "  - .agpr_count:     0\n    .name:           k2\n    .vgpr_count:     9\n"
           "amdhsa.target:   amdgcn-amd-amdhsa--gfx950\n    .name:           not_a_kernel\n")
    r = build.kernel_resources(asm)
    assert r == {"k1": {"agpr": 4, "lds": 1024, "scratch": 8, "sgpr": 20, "sgpr_spill": 0, "vgpr": 40,
                        "vgpr_spill": 2},
                 "k2": {"agpr": 0, "vgpr": 9}}


def _head_dim(name):
    m = re.search(r"kernelILi(\d+)E", name)
    return int(m.group(1)) if m else None


def test_hot_kernels_fit_their_register_budgets(built):
    """Two waves per SIMD (eight-wave workgroups, or two four-wave workgroups per CU) need
    at most 256 registers (VGPR + AGPR) a lane; spills to scratch memory are confined to
    the precise d = 256 path and the paired two-group form at d = 128 (a few registers,
    stored before the tile loops and reloaded once per item); every kernel fits the
    160 KiB of LDS of a CU."""
    pre = build.kernel_resources(build.device_asm("prefill.hip", built))
    dec = build.kernel_resources(build.device_asm("decode.hip", built))
    narrow = [k for k in pre if "prefill_narrow_kernel" in k]
    main = [k for k in pre if "14prefill_kernel" in k]
    assert len(narrow) == 2 and len(main) == 30     # d = 256 main kernel: precise only; eight waves: d = 128
    for k in narrow:
        r = pre[k]
        assert r["vgpr_spill"] == 0 and r["scratch"] == 0, (k, r)
        assert r["vgpr"] + r["agpr"] <= 256, (k, r)
    for k in main:
        r, d = pre[k], _head_dim(k)
        if d == 256:
            continue                     # precise d = 256: one wave per SIMD, 512 registers
        assert r["vgpr"] + r["agpr"] <= 256, (k, r)
        paired = k.endswith("Lb1EEEvNS_13PrefillParamsE")
        assert r["vgpr_spill"] <= (8 if d == 128 and paired else 0), (k, r)
    for k, r in dec.items():
        assert r["vgpr_spill"] == 0 and r["scratch"] == 0, (k, r)
    for k, r in {**pre, **dec}.items():
        assert r["lds"] <= 160 * 1024, (k, r)


def _kernel_bodies(asm):
    """{mangled kernel name: its instructions, in order} from gfx950 assembly."""
    out, name, body = {}, None, []
    for line in asm.split("\n"):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        if line.startswith(".Lfunc_end"):
            out[name], name = body, None
            continue
        t = line.strip()
        if t and not t.startswith((";", ".")):
            body.append(t.split()[0])
    return out


@pytest.fixture(scope="module")
def built_poison(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("asm_poison"))
    build.compile_all(d, jobs=3, defines=("-DATTN_POISON_LDS=1",))
    return d


def test_poison_build_fills_lds_before_any_copy_or_read(built, built_poison):
    """In the LDS-poisoning debug build every kernel that uses LDS stores to it and passes
    a barrier before its first global->LDS copy or LDS read; the LDS sizes and the set of
    kernels are those of the release build."""
    for src in ("prefill.hip", "decode.hip"):
        rel = build.kernel_resources(build.device_asm(src, built))
        asm = build.device_asm(src, built_poison)
        dbg = build.kernel_resources(asm)
        assert set(dbg) == set(rel), src
        bodies = _kernel_bodies(asm)
        with_lds = [k for k, r in dbg.items() if r.get("lds", 0) > 0]
        assert with_lds, src
        for k in with_lds:
            assert dbg[k]["lds"] == rel[k]["lds"], k
            ins = bodies[k]
            first = next(i for i, x in enumerate(ins)
                         if x.startswith(("ds_read", "global_load_lds", "buffer_load")) and
                         (x.startswith("ds_read") or "lds" in x))
            head = ins[:first]
            assert any(x.startswith("ds_write") for x in head), k
            assert "s_barrier" in head, k
