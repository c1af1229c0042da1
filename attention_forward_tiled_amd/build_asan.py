"""AddressSanitizer build of libattn.so's host code, for the CPU tests of the C ABI.

    python -m attention_forward_tiled_amd.build_asan OUT_DIR

The host side of attn_api.cpp (argument validation, workspace layout, error
reporting) is compiled with AddressSanitizer; the kernels' device code is built as
usual (no GPU sanitizer). The library links the sanitizer runtime dynamically, so a
process that loads it must have ``libclang_rt.asan`` preloaded (``asan_runtime()``).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from .build import ARCH, CSRC, EXTRA_FLAGS, SOURCES, flags, hipcc

_HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that matches hipcc."""
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cands = sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    cands += sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not cands:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found next to hipcc")
    return cands[-1]


def build_asan(out_dir: str, jobs: int = 3) -> str:
    os.makedirs(out_dir, exist_ok=True)

    def one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        extra = _HOST_ASAN if src.endswith(".cpp") else []
        cmd = [hipcc(), *flags(), *EXTRA_FLAGS.get(src, []), *extra, "-x", "hip", "-c",
               os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(one, SOURCES))
    out = os.path.join(out_dir, "libattn_asan.so")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-shared-libasan", "-o", out, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    return out


if __name__ == "__main__":
    print(build_asan(sys.argv[1] if len(sys.argv) > 1 else "_build/asan"))
