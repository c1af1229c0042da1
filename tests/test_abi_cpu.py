"""The C ABI without a GPU: every declared symbol is exported, and invalid
arguments are rejected on the host with the documented status and a message."""
import ctypes
import os
import re

import pytest

from attention_forward_tiled_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "attn.h")).read()
    return sorted(set(re.findall(r"^\s*(?:[a-z_0-9]+\s*\*?\s+)+(attn_[a-z_0-9]+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_symbols_exported(lib):
    names = header_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_poison_build_exports_the_same_symbols():
    # the LDS-poisoning debug build is the same source compiled with one define
    dbg = _lib.open_library(_lib.POISON_LIB_PATH)
    for n in header_functions():
        assert hasattr(dbg, n), n
    assert dbg.attn_abi_version() == _lib.ATTN_ABI_VERSION


def test_abi_version(lib):
    assert lib.attn_abi_version() == _lib.ATTN_ABI_VERSION


def test_header_constants_match_binding():
    text = open(os.path.join(ROOT, "include", "attn.h")).read()
    assert f"#define ATTN_PAGE_SIZE {_lib.ATTN_PAGE_SIZE} " in text
    assert f"#define ATTN_MAX_SPLITS {_lib.ATTN_MAX_SPLITS} " in text
    assert f"#define ATTN_MAX_SEQLEN (1 << {_lib.ATTN_MAX_SEQLEN.bit_length() - 1})" in text
    assert f"#define ATTN_ABI_VERSION {_lib.ATTN_ABI_VERSION}" in text
    assert f"#define ATTN_NOALLOC_SCRATCH_BYTES ({_lib.ATTN_NOALLOC_SCRATCH_BYTES >> 20}u << 20)" in text


def test_struct_sizes():
    # the ctypes mirrors must have the C layout (all fields naturally aligned, no padding holes)
    assert ctypes.sizeof(_lib.PrefillArgs) == 8 * 8 + 16 * 4 + 8 + 8   # workspace pointer and size last
    assert _lib.PrefillArgs.workspace.offset == 128 and _lib.PrefillArgs.kv_splits.offset == 124
    assert ctypes.sizeof(_lib.DecodeArgs) == 8 * 8 + 8 + 12 * 4
    assert ctypes.sizeof(_lib.CombineArgs) == 4 * 8 + 6 * 4
    assert ctypes.sizeof(_lib.DeviceInfo) == 2 * 256 + 8 + 8 * 4


FAKE = 0x1000  # aligned non-null pointer value; never dereferenced (validation fails first)


def prefill_args(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, block_table=FAKE, seqlens_k=FAKE, cu_seqlens_q=None,
             batch=1, num_heads_q=4, num_heads_kv=2, seqlen_q=128, seqlen_k=128, head_dim=128,
             num_blocks=2, max_blocks_per_seq=2, qkv_dtype=_lib.ATTN_F16, o_dtype=_lib.ATTN_F16,
             layout=_lib.ATTN_BSHD, causal=1, precise=0, scale=0.0, o_round=_lib.ATTN_ROUND_RTNE,
             kv_splits=0, workspace=None, workspace_bytes=0)
    a.update(kw)
    return _lib.PrefillArgs(**a)


def decode_args(**kw):
    a = dict(q=FAKE, k_cache=FAKE, v_cache=FAKE, block_table=FAKE, seqlens_k=FAKE, o=FAKE, lse=None,
             workspace=FAKE, workspace_bytes=1 << 30, batch=2, num_heads_q=8, num_heads_kv=2,
             head_dim=128, num_blocks=10, max_blocks_per_seq=5, max_seqlen_k=300, num_splits=4,
             qkv_dtype=_lib.ATTN_BF16, o_dtype=_lib.ATTN_BF16, scale=0.0, o_round=_lib.ATTN_ROUND_RTNE)
    a.update(kw)
    return _lib.DecodeArgs(**a)


def combine_args(**kw):
    a = dict(partial_o=FAKE, partial_lse=FAKE, o=FAKE, lse=None, batch=2, num_heads=4, num_splits=8,
             head_dim=128, o_dtype=_lib.ATTN_F32, o_round=_lib.ATTN_ROUND_RTNE)
    a.update(kw)
    return _lib.CombineArgs(**a)


BAD_PREFILL = [
    (dict(head_dim=96), _lib.ATTN_ERR_INVALID_ARG, "head_dim"),
    (dict(num_heads_q=5, num_heads_kv=2), _lib.ATTN_ERR_INVALID_ARG, "multiple"),
    (dict(num_heads_kv=0), _lib.ATTN_ERR_INVALID_ARG, "positive"),
    (dict(qkv_dtype=_lib.ATTN_F32), _lib.ATTN_ERR_INVALID_ARG, "qkv_dtype"),
    (dict(o_dtype=7), _lib.ATTN_ERR_INVALID_ARG, "o_dtype"),
    (dict(layout=2), _lib.ATTN_ERR_INVALID_ARG, "layout"),
    (dict(causal=2), _lib.ATTN_ERR_INVALID_ARG, "causal"),
    (dict(q=None), _lib.ATTN_ERR_INVALID_ARG, "non-NULL"),
    (dict(o=FAKE + 2), _lib.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(seqlens_k=None), _lib.ATTN_ERR_INVALID_ARG, "seqlens_k"),
    (dict(max_blocks_per_seq=1), _lib.ATTN_ERR_INVALID_ARG, "fewer than seqlen_k"),
    (dict(scale=float("nan")), _lib.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(num_heads_q=258, num_heads_kv=2), _lib.ATTN_ERR_UNSUPPORTED, "GQA"),
    (dict(batch=-1), _lib.ATTN_ERR_INVALID_ARG, "batch"),
    (dict(seqlen_q=(1 << 30) + 1), _lib.ATTN_ERR_UNSUPPORTED, "seqlen_q and seqlen_k must be <="),
    (dict(seqlen_k=(1 << 30) + 1, max_blocks_per_seq=(1 << 24) + 1), _lib.ATTN_ERR_UNSUPPORTED,
     "seqlen_q and seqlen_k must be <="),
    (dict(o_round=3), _lib.ATTN_ERR_INVALID_ARG, "o_round"),
    (dict(o_round=_lib.ATTN_ROUND_RTZ), _lib.ATTN_ERR_UNSUPPORTED, "fp16"),     # fp16 output
    (dict(cu_seqlens_q=FAKE, layout=_lib.ATTN_BHSD), _lib.ATTN_ERR_INVALID_ARG, "BSHD"),
    (dict(cu_seqlens_q=FAKE + 2), _lib.ATTN_ERR_INVALID_ARG, "cu_seqlens_q"),
    (dict(kv_splits=-1), _lib.ATTN_ERR_INVALID_ARG, "kv_splits"),
    (dict(kv_splits=65), _lib.ATTN_ERR_INVALID_ARG, "kv_splits"),
    (dict(kv_splits=4), _lib.ATTN_ERR_INVALID_ARG, "needs a workspace"),
    (dict(workspace=FAKE + 16, workspace_bytes=1 << 20), _lib.ATTN_ERR_INVALID_ARG, "256-byte"),
    (dict(workspace_bytes=64), _lib.ATTN_ERR_INVALID_ARG, "without a workspace"),
]


@pytest.mark.parametrize("kw,status,msg", BAD_PREFILL, ids=lambda x: str(x)[:40])
def test_prefill_rejects(lib, kw, status, msg):
    st = lib.attn_prefill_fwd(ctypes.byref(prefill_args(**kw)), None)
    assert st == status
    assert msg in _lib.last_error()


def test_null_args_pointer(lib):
    assert lib.attn_prefill_fwd(None, None) == _lib.ATTN_ERR_INVALID_ARG
    assert lib.attn_decode_fwd(None, None) == _lib.ATTN_ERR_INVALID_ARG
    assert lib.attn_splitkv_combine(None, None) == _lib.ATTN_ERR_INVALID_ARG
    assert lib.attn_device_info(0, None) == _lib.ATTN_ERR_INVALID_ARG
    assert "NULL" in _lib.last_error()


def test_device_info_rejects_negative_index(lib):
    info = _lib.DeviceInfo()
    assert lib.attn_device_info(-1, ctypes.byref(info)) == _lib.ATTN_ERR_INVALID_ARG
    assert "device" in _lib.last_error()


def test_prefill_workspace_query_without_device(lib):
    # a size query: 0 for arguments the call would reject, for kv_splits = 1 and (here,
    # with no device to plan on) for everything else; it leaves the last error alone
    assert lib.attn_prefill_fwd(ctypes.byref(prefill_args(head_dim=96)), None) == _lib.ATTN_ERR_INVALID_ARG
    before = _lib.last_error()
    assert lib.attn_prefill_workspace_bytes(ctypes.byref(prefill_args(kv_splits=1, causal=0))) == 0
    assert lib.attn_prefill_workspace_bytes(ctypes.byref(prefill_args(kv_splits=99))) == 0
    assert lib.attn_prefill_workspace_bytes(None) == 0
    if lib.attn_device_count() == 0:
        assert lib.attn_prefill_workspace_bytes(ctypes.byref(prefill_args(kv_splits=4, causal=0))) == 0
    assert _lib.last_error() == before


def test_prefill_empty_is_noop(lib):
    assert lib.attn_prefill_fwd(ctypes.byref(prefill_args(batch=0, q=None)), None) == _lib.ATTN_OK
    assert lib.attn_prefill_fwd(ctypes.byref(prefill_args(seqlen_q=0, q=None)), None) == _lib.ATTN_OK
    assert _lib.last_error() == ""


BAD_DECODE = [
    (dict(num_splits=0), _lib.ATTN_ERR_INVALID_ARG, "num_splits"),
    (dict(num_splits=65), _lib.ATTN_ERR_INVALID_ARG, "num_splits"),
    (dict(num_heads_q=64, num_heads_kv=2), _lib.ATTN_ERR_UNSUPPORTED, "GQA"),
    (dict(workspace_bytes=16), _lib.ATTN_ERR_INVALID_ARG, "workspace"),
    (dict(workspace=FAKE + 16), _lib.ATTN_ERR_INVALID_ARG, "256-byte"),
    (dict(max_seqlen_k=321), _lib.ATTN_ERR_INVALID_ARG, "fewer than max_seqlen_k"),
    (dict(max_seqlen_k=(1 << 30) + 1, max_blocks_per_seq=(1 << 24) + 1), _lib.ATTN_ERR_UNSUPPORTED,
     "max_seqlen_k must be <="),
    (dict(block_table=None), _lib.ATTN_ERR_INVALID_ARG, "non-NULL"),
    (dict(head_dim=32), _lib.ATTN_ERR_INVALID_ARG, "head_dim"),
    (dict(qkv_dtype=_lib.ATTN_F32), _lib.ATTN_ERR_INVALID_ARG, "qkv_dtype"),
    (dict(o_round=-1), _lib.ATTN_ERR_INVALID_ARG, "o_round"),
    (dict(o_dtype=_lib.ATTN_F16, o_round=_lib.ATTN_ROUND_RTNA), _lib.ATTN_ERR_UNSUPPORTED, "fp16"),
]


@pytest.mark.parametrize("kw,status,msg", BAD_DECODE, ids=lambda x: str(x)[:40])
def test_decode_rejects(lib, kw, status, msg):
    st = lib.attn_decode_fwd(ctypes.byref(decode_args(**kw)), None)
    assert st == status
    assert msg in _lib.last_error()


@pytest.mark.parametrize("kw,msg", [(dict(num_splits=0), "num_splits"), (dict(head_dim=100), "head_dim"),
                                    (dict(o_dtype=3), "o_dtype"), (dict(partial_o=None), "non-NULL"),
                                    (dict(o_round=5), "o_round")])
def test_combine_rejects(lib, kw, msg):
    assert lib.attn_splitkv_combine(ctypes.byref(combine_args(**kw)), None) == _lib.ATTN_ERR_INVALID_ARG
    assert msg in _lib.last_error()


def test_decode_noalloc_rejects(lib):
    # the allocation-free decode takes no workspace, and refuses sizes whose partials and
    # plan would not fit its static scratch; both are host-side checks
    st = lib.attn_decode_fwd_noalloc(ctypes.byref(decode_args()), None)
    assert st == _lib.ATTN_ERR_INVALID_ARG and "takes no workspace" in _lib.last_error()
    big = decode_args(workspace=None, workspace_bytes=0, batch=64, num_heads_q=64, num_heads_kv=8,
                      num_splits=16)      # 64 * 64 * 16 * 128 * 4 bytes = 32 MiB of partials + plan
    need = lib.attn_decode_workspace_bytes(64, 64, 16, 128)
    assert need > _lib.ATTN_NOALLOC_SCRATCH_BYTES
    st = lib.attn_decode_fwd_noalloc(ctypes.byref(big), None)
    assert st == _lib.ATTN_ERR_INVALID_ARG and "maximum" in _lib.last_error()
    st = lib.attn_decode_fwd_noalloc(ctypes.byref(decode_args(workspace=None, workspace_bytes=0, num_splits=0)),
                                     None)
    assert st == _lib.ATTN_ERR_INVALID_ARG and "num_splits" in _lib.last_error()


def test_workspace_bytes(lib):
    n = lib.attn_decode_workspace_bytes(32, 32, 16, 128)
    assert n >= 32 * 32 * 16 * 129 * 4 and n % 256 == 0
    assert lib.attn_decode_workspace_bytes(1, 1, 65, 128) == 0
    assert lib.attn_decode_workspace_bytes(1, 1, 1, 100) == 0


@pytest.mark.skipif(_lib.load().attn_device_count() > 0, reason="a GPU is present; fake pointers must not launch")
def test_valid_call_without_device_reports_no_device(lib):
    assert lib.attn_prefill_fwd(ctypes.byref(prefill_args()), None) == _lib.ATTN_ERR_NO_DEVICE
    assert lib.attn_decode_fwd(ctypes.byref(decode_args()), None) == _lib.ATTN_ERR_NO_DEVICE
    assert lib.attn_splitkv_combine(ctypes.byref(combine_args()), None) == _lib.ATTN_ERR_NO_DEVICE
    assert lib.attn_device_info(0, ctypes.byref(_lib.DeviceInfo())) == _lib.ATTN_ERR_NO_DEVICE
    fits = decode_args(workspace=None, workspace_bytes=0)
    assert lib.attn_decode_fwd_noalloc(ctypes.byref(fits), None) == _lib.ATTN_ERR_NO_DEVICE


def test_missing_library_raises(tmp_path, monkeypatch):
    """No fallback: with libattn.so absent, the binding refuses to run at all."""
    from attention_forward_tiled_amd import _lib
    monkeypatch.setattr(_lib, "_LIB", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libattn.so"))
    monkeypatch.setattr(_lib.load, "__defaults__", (str(tmp_path / "libattn.so"),))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load()
    from attention_forward_tiled_amd import attn_decode_workspace_bytes
    with pytest.raises(RuntimeError, match="not built"):
        attn_decode_workspace_bytes(1, 4, 2, 64)


def test_bench_refuses_more_than_one_gpu():
    # one GPU only: a request for several exits non-zero with a message, before any
    # device work
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU only" in (r.stdout + r.stderr)
    assert r.stdout.strip() == "" or not r.stdout.lstrip().startswith("{")


def test_bench_worst_samples_names_the_deviations():
    # --debug-mismatch: the largest deviations, worst first, with each index mapped back to
    # the whole output where the parity sample took a subset of the query rows
    import sys
    sys.path.insert(0, ROOT)
    import numpy as np
    from bench import worst_samples
    rows = np.array([3, 40, 77])
    ref = np.zeros((2, 3, 4, 8))           # [seq, sampled row, head, col]
    got = ref.copy()
    got[1, 2, 3, 5] = 0.5
    got[0, 1, 0, 0] = -0.25
    got[1, 0, 2, 7] = 1e-3
    w = worst_samples(got, ref, 2, ("seq", "row", "head", "col"), (None, rows, None, None))
    assert [(x["seq"], x["row"], x["head"], x["col"]) for x in w] == [(1, 77, 3, 5), (0, 40, 0, 0)]
    assert w[0]["got"] == 0.5 and w[0]["expected"] == 0.0 and w[1]["abs_err"] == 0.25
