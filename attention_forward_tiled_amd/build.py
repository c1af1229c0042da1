"""Build libattn.so (gfx950) in-tree with hipcc.

    python -m attention_forward_tiled_amd.build [--jobs N]

Every HIP source is compiled for gfx950 only. Packed fp32 VALU instructions are
disabled on purpose (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
Objects go to ``_build/``; the shared library lands next to this file. A second,
debug library, ``libattn_poison.so`` (objects in ``_build/poison``), is the same code
compiled with ``-DATTN_POISON_LDS=1``: every kernel first fills its LDS with NaN bit
patterns, so that a test run against it shows any read of LDS that nothing wrote.

The kernels issue their global->LDS copies (global_load_lds_dwordx4) from inline asm
that sets m0, the LDS destination register, without the compiler knowing (the
compiler reserves m0 and cannot take it as a clobber). That is only correct while the
generated code keeps nothing of its own in m0. Every build therefore keeps the gfx950
assembly (``-save-temps=obj``) and checks it: m0 may appear only as the destination of
the ``s_mov_b32 m0, sN`` that directly precedes such a copy, and no instruction that
reads m0 implicitly (register-indexed moves, messages, GWS) may appear. The build fails
otherwise.
"""
from __future__ import annotations

import argparse
import glob
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libattn.so")
OUT_POISON = os.path.join(HERE, "libattn_poison.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["attn_api.cpp", "prefill.hip", "decode.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libattn.so")


def flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Wno-unused-lambda-capture", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]


# Per-source additions. The prefill tile loop takes per-lane maxima of its scores on every
# tile; no NaN can reach them (masked scores are -inf and key rows past a sequence's
# length are read from a zero block), so the compiler is told it need not quiet
# signalling NaNs before each max (one instruction per two scores saved).
EXTRA_FLAGS = {"prefill.hip": ["-fno-honor-nans"]}


# Instructions that read or write m0 implicitly on gfx9-family targets.
_M0_IMPLICIT = re.compile(r"^\s*(s_movrel\w*|v_movrel\w*|s_set_gpr_idx_\w*|s_sendmsg\w*|ds_gws_\w*|"
                          r"v_interp\w*|buffer_\w+\s.*\blds\b)")
_M0 = re.compile(r"\bm0\b")


def check_m0(asm: str) -> list:
    """Uses of m0 in gfx950 assembly other than the LDS-copy idiom
    ``s_mov_b32 m0, sN`` / ``s_nop 0`` / ``global_load_lds_dwordx4``; returns the offending
    lines (empty when the invariant holds)."""
    lines = [l.split(";", 1)[0].rstrip() for l in asm.splitlines()]
    code = [(i, l.strip()) for i, l in enumerate(lines) if l.strip() and not l.strip().startswith((".", "//"))
            and not l.strip().endswith(":")]
    bad = []
    for n, (i, l) in enumerate(code):
        if _M0_IMPLICIT.match(l):
            bad.append(f"line {i + 1}: {l}")
        elif _M0.search(l):
            ok = (re.fullmatch(r"s_mov_b32\s+m0,\s*s\d+", l) is not None and n + 2 < len(code)
                  and code[n + 1][1] == "s_nop 0" and code[n + 2][1].startswith("global_load_lds_dwordx4"))
            if not ok:
                bad.append(f"line {i + 1}: {l}")
    return bad


def _compile(src: str, build_dir: str = BUILD, defines: tuple = ()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *flags(), *EXTRA_FLAGS.get(src, []), *defines, "-save-temps=obj", "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=build_dir)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def device_asm(src: str, build_dir: str = BUILD) -> str:
    """The gfx950 assembly that the last compile of `src` left in `build_dir`."""
    stem = os.path.splitext(src)[0]
    paths = glob.glob(os.path.join(build_dir, f"{stem}-hip-amdgcn-amd-amdhsa-{ARCH}*.s"))
    if len(paths) != 1:
        raise RuntimeError(f"expected one {ARCH} assembly file for {src} in {build_dir}, found {paths}")
    with open(paths[0]) as f:
        return f.read()


def kernel_resources(asm: str) -> dict:
    """Per-kernel resource figures from the code-object metadata of gfx950 assembly:
    {mangled name: {"vgpr", "agpr", "sgpr", "vgpr_spill", "sgpr_spill", "lds", "scratch"}}."""
    keys = {".vgpr_count": "vgpr", ".agpr_count": "agpr", ".sgpr_count": "sgpr", ".vgpr_spill_count": "vgpr_spill",
            ".sgpr_spill_count": "sgpr_spill", ".group_segment_fixed_size": "lds",
            ".private_segment_fixed_size": "scratch"}
    out, cur, inside = {}, None, False
    for line in asm.splitlines():
        if line.startswith("amdhsa.kernels:"):
            inside = True
            continue
        if not inside:
            continue
        if line and not line.startswith(" "):
            break                       # the next top-level key ends the kernel list
        if line.startswith("  - "):
            cur = {}
            line = "    " + line[4:]
        if cur is None or not line.startswith("    ."):
            continue
        key, _, val = line.strip().partition(":")
        if key == ".name":
            out[val.strip()] = cur
        elif key in keys:
            cur[keys[key]] = int(val)
    return out


def compile_all(build_dir: str = BUILD, jobs: int = 4, defines: tuple = ()) -> list:
    """Compile every source into `build_dir` and check the m0 invariant of its assembly."""
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, defines), SOURCES))
    for src in SOURCES:
        bad = check_m0(device_asm(src, build_dir))
        if bad:
            raise RuntimeError(f"{src}: m0 used outside the LDS-copy idiom (the inline-asm copies would "
                               "clobber it):\n  " + "\n  ".join(bad[:20]))
    return objs


def _link(objs: list, out: str, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def build(jobs: int = 4, verbose: bool = True, poison: bool = True) -> str:
    """Build libattn.so and (poison=True) the LDS-poisoning debug library beside it."""
    out = _link(compile_all(BUILD, jobs), OUT, verbose)
    if poison:
        _link(compile_all(os.path.join(BUILD, "poison"), jobs, ("-DATTN_POISON_LDS=1",)), OUT_POISON, verbose)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--no-poison", action="store_true", help="skip the LDS-poisoning debug library")
    a = ap.parse_args()
    build(a.jobs, poison=not a.no_poison)
