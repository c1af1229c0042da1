"""The m0 invariant of the inline-asm LDS copies, checked on freshly compiled gfx950
assembly (CPU only: hipcc cross-compiles), and the checker itself on small samples."""
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


def test_compiled_kernels_keep_m0_for_the_copies(tmp_path):
    # compile_all raises if any source's gfx950 assembly uses m0 outside the idiom
    build.compile_all(str(tmp_path), jobs=3)
    asm = build.device_asm("prefill.hip", str(tmp_path))
    assert asm.count("global_load_lds_dwordx4") > 0
    assert build.check_m0(asm) == []
