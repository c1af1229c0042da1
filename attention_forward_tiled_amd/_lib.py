"""ctypes view of libattn.so: the structures and prototypes of include/attn.h.

Loading fails loudly when the library has not been built: there is no fallback
implementation anywhere in this package.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_LAUNCH, ATTN_ERR_NO_DEVICE = range(5)
STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "LAUNCH", 4: "NO_DEVICE"}
ATTN_F16, ATTN_BF16, ATTN_F32 = 0, 1, 2
ATTN_BSHD, ATTN_BHSD = 0, 1
ATTN_ROUND_RTNE, ATTN_ROUND_RTNA, ATTN_ROUND_RTZ = 0, 1, 2
ATTN_PAGE_SIZE = 64
ATTN_MAX_SPLITS = 64
ATTN_MAX_SEQLEN = 1 << 30
ATTN_NOALLOC_SCRATCH_BYTES = 32 << 20
ATTN_ABI_VERSION = 5

EXPORTS = ("attn_prefill_fwd", "attn_decode_fwd", "attn_decode_workspace_bytes",
           "attn_splitkv_combine", "attn_last_error", "attn_abi_version", "attn_device_count",
           "attn_device_info", "attn_decode_fwd_noalloc", "attn_prefill_workspace_bytes")

_c_void_p, _i32, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float


class PrefillArgs(ctypes.Structure):
    _fields_ = [("q", _c_void_p), ("k", _c_void_p), ("v", _c_void_p), ("o", _c_void_p),
                ("lse", _c_void_p), ("block_table", _c_void_p), ("seqlens_k", _c_void_p),
                ("cu_seqlens_q", _c_void_p),
                ("batch", _i32), ("num_heads_q", _i32), ("num_heads_kv", _i32),
                ("seqlen_q", _i32), ("seqlen_k", _i32), ("head_dim", _i32),
                ("num_blocks", _i32), ("max_blocks_per_seq", _i32),
                ("qkv_dtype", _i32), ("o_dtype", _i32), ("layout", _i32),
                ("causal", _i32), ("precise", _i32), ("scale", _f32), ("o_round", _i32),
                ("kv_splits", _i32), ("workspace", _c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("q", _c_void_p), ("k_cache", _c_void_p), ("v_cache", _c_void_p),
                ("block_table", _c_void_p), ("seqlens_k", _c_void_p), ("o", _c_void_p),
                ("lse", _c_void_p), ("workspace", _c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("batch", _i32), ("num_heads_q", _i32), ("num_heads_kv", _i32), ("head_dim", _i32),
                ("num_blocks", _i32), ("max_blocks_per_seq", _i32), ("max_seqlen_k", _i32),
                ("num_splits", _i32), ("qkv_dtype", _i32), ("o_dtype", _i32), ("scale", _f32),
                ("o_round", _i32)]


class CombineArgs(ctypes.Structure):
    _fields_ = [("partial_o", _c_void_p), ("partial_lse", _c_void_p), ("o", _c_void_p),
                ("lse", _c_void_p), ("batch", _i32), ("num_heads", _i32), ("num_splits", _i32),
                ("head_dim", _i32), ("o_dtype", _i32), ("o_round", _i32)]


class DeviceInfo(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 256), ("arch", ctypes.c_char * 256),
                ("total_memory", ctypes.c_int64), ("compute_units", _i32), ("clock_khz", _i32),
                ("memory_clock_khz", _i32), ("memory_bus_bits", _i32), ("lds_per_cu", _i32),
                ("l2_bytes", _i32), ("runtime_version", _i32), ("driver_version", _i32)]


_LIB = None
POISON_LIB_PATH = os.path.join(HERE, "libattn_poison.so")   # debug build: LDS filled with NaN first


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libattn.so once; raise if it is missing or its ABI version differs."""
    global _LIB
    if _LIB is not None:
        return _LIB
    _LIB = open_library(path)
    return _LIB


def open_library(path: str) -> ctypes.CDLL:
    """Open a build of the library (libattn.so, or the LDS-poisoning debug build) with the
    prototypes of include/attn.h; raise if it is missing or its ABI version differs."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m attention_forward_tiled_amd.build` "
            "(the HIP library is the only implementation)")
    lib = ctypes.CDLL(path)
    lib.attn_prefill_fwd.argtypes = [ctypes.POINTER(PrefillArgs), _c_void_p]
    lib.attn_prefill_fwd.restype = ctypes.c_int
    lib.attn_prefill_workspace_bytes.argtypes = [ctypes.POINTER(PrefillArgs)]
    lib.attn_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_decode_fwd.argtypes = [ctypes.POINTER(DecodeArgs), _c_void_p]
    lib.attn_decode_fwd.restype = ctypes.c_int
    lib.attn_decode_fwd_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), _c_void_p]
    lib.attn_decode_fwd_noalloc.restype = ctypes.c_int
    lib.attn_splitkv_combine.argtypes = [ctypes.POINTER(CombineArgs), _c_void_p]
    lib.attn_splitkv_combine.restype = ctypes.c_int
    lib.attn_decode_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32]
    lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = _i32
    lib.attn_device_count.argtypes = []
    lib.attn_device_count.restype = _i32
    lib.attn_device_info.argtypes = [_i32, ctypes.POINTER(DeviceInfo)]
    lib.attn_device_info.restype = ctypes.c_int
    if lib.attn_abi_version() != ATTN_ABI_VERSION:
        raise RuntimeError(f"{os.path.basename(path)} ABI version {lib.attn_abi_version()} != {ATTN_ABI_VERSION}")
    return lib


def last_error() -> str:
    return load().attn_last_error().decode()
