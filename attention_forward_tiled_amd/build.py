"""Build libattn.so (gfx950) in-tree with hipcc.

    python -m attention_forward_tiled_amd.build [--jobs N]

Every HIP source is compiled for gfx950 only. Packed fp32 VALU instructions are
disabled on purpose (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
Objects go to ``_build/``; the shared library lands next to this file.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libattn.so")
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


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *flags(), *EXTRA_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 4, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    build(ap.parse_args().jobs)
