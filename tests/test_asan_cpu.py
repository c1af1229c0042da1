"""The C ABI's host code under AddressSanitizer (CPU only).

attn_api.cpp is built with -fsanitize=address (host side) into a separate library,
and the whole C-ABI test module runs against it in a child process that has the
sanitizer runtime preloaded: every validation path, the no-device path and the
workspace arithmetic then run with heap, stack and global bounds checked.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = """
import sys
sys.path.insert(0, {root!r})
from attention_forward_tiled_amd import _lib
lib = _lib.load({lib!r})
import ctypes
assert hasattr(ctypes.CDLL(None), "__asan_init"), "sanitizer runtime not loaded"
import pytest
sys.exit(int(pytest.main(["-q", "-x", "-p", "no:cacheprovider", {tests!r}])))
"""


def test_abi_under_address_sanitizer(tmp_path):
    from attention_forward_tiled_amd.build_asan import asan_runtime, build_asan
    lib = build_asan(str(tmp_path))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms, "host code is not instrumented"
    env = dict(os.environ, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:detect_odr_violation=0:abort_on_error=0:exitcode=99")
    code = DRIVER.format(root=ROOT, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi_cpu.py"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=600,
                       cwd=str(tmp_path))
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
