"""MI355X (gfx950) tiled attention forward.

The computation lives in ``libattn.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/attn.h``). This package is a thin binding: ``_lib`` mirrors
the C structures with ctypes and ``api`` marshals torch tensors (device memory
and the current stream) into those calls. There is no other implementation:
every entry point loads the library on first use and raises if it is not built
(``python -m attention_forward_tiled_amd.build``).
"""
from .api import (  # noqa: F401
    AttnError,
    attn_decode_fwd,
    attn_decode_fwd_noalloc,
    attn_decode_workspace_bytes,
    attn_device_info,
    attn_prefill_fwd,
    attn_prefill_workspace_bytes,
    attn_splitkv_combine,
)
from ._lib import load as load_library  # noqa: F401
