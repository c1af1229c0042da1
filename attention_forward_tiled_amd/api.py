"""Python binding over the C ABI, named like the C entry points.

Argument marshalling only: torch tensors supply device pointers and the current
HIP stream; every step of the computation runs in the HIP kernels of libattn.so.
Shapes are read from the tensors; the library re-validates everything.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib

_DT = {torch.float16: _lib.ATTN_F16, torch.bfloat16: _lib.ATTN_BF16, torch.float32: _lib.ATTN_F32}
_LAYOUT = {"bshd": _lib.ATTN_BSHD, "bhsd": _lib.ATTN_BHSD}
_ROUND = {"rtne": _lib.ATTN_ROUND_RTNE, "rtna": _lib.ATTN_ROUND_RTNA, "rtz": _lib.ATTN_ROUND_RTZ}


def _round(mode: str) -> int:
    if mode not in _ROUND:
        raise ValueError(f"out_round must be one of {sorted(_ROUND)}")
    return _ROUND[mode]


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_lib.STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(status: int):
    if status != _lib.ATTN_OK:
        raise AttnError(status, _lib.last_error())


def _need(t: torch.Tensor, name: str, dtypes=None, contiguous=True):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")


def attn_prefill_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool,
                     block_table: Optional[torch.Tensor] = None,
                     seqlens_k: Optional[torch.Tensor] = None, seqlen_k: Optional[int] = None,
                     layout: str = "bshd", out: Optional[torch.Tensor] = None,
                     out_dtype: Optional[torch.dtype] = None, lse: Optional[torch.Tensor] = None,
                     scale: float = 0.0, precise: bool = False, out_round: str = "rtne",
                     cu_seqlens_q: Optional[torch.Tensor] = None, max_seqlen_q: Optional[int] = None,
                     kv_splits: int = 0, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """Tiled attention forward. q: [B,S_q,Hq,d] (bshd) or [B,Hq,S_q,d] (bhsd).

    Paged K/V (block_table given): k, v are [num_blocks, 64, Hkv, d] caches and
    seqlens_k [B] int32 is required; ``seqlen_k`` (host-side bound) defaults to
    64 * block_table.shape[1]. Dense K/V: k, v in the layout of q.

    Packed queries: with ``cu_seqlens_q`` ([B+1] int32, first row of each sequence)
    q and the output are [total_q, Hq, d] and ``max_seqlen_q`` bounds the per-sequence
    query counts; lse, when given, is [Hq, total_q].

    Tail split (precise off): ``kv_splits`` 0 lets the library split the key range of
    the last round of work items when that round would leave half of the CUs idle
    (non-causal), or of every item when a causal launch has that few items;
    1 turns it off, n >= 2 splits those items into n parts. The partials go to ``workspace``
    (uint8 device tensor of at least attn_prefill_workspace_bytes bytes), allocated here
    when the call needs one and none is given.
    """
    _need(q, "q", (torch.float16, torch.bfloat16))
    _need(k, "k", (q.dtype,))
    _need(v, "v", (q.dtype,))
    if k.dim() != 4 or v.shape != k.shape:
        raise ValueError("k and v must be 4-D tensors of the same shape")
    if layout not in _LAYOUT:
        raise ValueError("layout must be 'bshd' or 'bhsd'")
    if cu_seqlens_q is not None:
        _need(cu_seqlens_q, "cu_seqlens_q", (torch.int32,))
        if q.dim() != 3 or layout != "bshd":
            raise ValueError("packed queries: q must be [total_q, Hq, d] (bshd)")
        if max_seqlen_q is None:
            raise ValueError("packed queries need max_seqlen_q")
        B, (_, Hq, d), Sq = cu_seqlens_q.numel() - 1, q.shape, int(max_seqlen_q)
    elif q.dim() != 4:
        raise ValueError("q must be 4-D")
    elif layout == "bshd":
        B, Sq, Hq, d = q.shape
    else:
        B, Hq, Sq, d = q.shape
    paged = block_table is not None
    if k.shape[3] != d:
        raise ValueError("k and v must have the head size of q")
    if paged:
        _need(block_table, "block_table", (torch.int32,))
        if seqlens_k is None:
            raise ValueError("paged K/V needs seqlens_k")
        if block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be [batch, max_blocks_per_seq]")
        num_blocks, page, Hkv = k.shape[0], k.shape[1], k.shape[2]
        if page != _lib.ATTN_PAGE_SIZE:
            raise ValueError(f"pages must hold {_lib.ATTN_PAGE_SIZE} tokens")
        max_blocks = block_table.shape[1]
        Sk = seqlen_k if seqlen_k is not None else max_blocks * _lib.ATTN_PAGE_SIZE
    else:
        num_blocks = max_blocks = 0
        if k.shape[0] != B:
            raise ValueError("dense K/V must have the batch of q")
        if layout == "bshd":
            Sk, Hkv = k.shape[1], k.shape[2]
        else:
            Hkv, Sk = k.shape[1], k.shape[2]
        if seqlen_k is not None and seqlen_k != Sk:
            raise ValueError("dense K/V: seqlen_k must equal the K/V row count")
    if seqlens_k is not None:
        _need(seqlens_k, "seqlens_k", (torch.int32,))
        if seqlens_k.numel() != B:
            raise ValueError("seqlens_k must hold one length per sequence")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out", tuple(_DT))
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    if lse is not None:
        _need(lse, "lse", (torch.float32,))
        want = (Hq, q.shape[0]) if cu_seqlens_q is not None else (B, Hq, Sq)
        if tuple(lse.shape) != want:
            raise ValueError(f"lse must be {list(want)}")
    a = _lib.PrefillArgs(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(block_table), _ptr(seqlens_k),
        _ptr(cu_seqlens_q), B, Hq, Hkv, Sq, Sk, d, num_blocks, max_blocks, _DT[q.dtype], _DT[out.dtype],
        _LAYOUT[layout], int(bool(causal)), int(bool(precise)), float(scale), _round(out_round),
        int(kv_splits), None, 0)
    lib = _lib.load()
    if workspace is None and int(kv_splits) != 1:
        need = int(lib.attn_prefill_workspace_bytes(ctypes.byref(a)))
        if need == 0 and int(kv_splits) >= 2:
            need = 256        # the C ABI takes a workspace with every kv_splits >= 2, split or not
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace", (torch.uint8,))
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    _check(lib.attn_prefill_fwd(ctypes.byref(a), _stream(stream)))
    return out


def attn_prefill_workspace_bytes(q: torch.Tensor, *, num_heads_kv: int, seqlen_k: int, causal: bool,
                                 layout: str = "bshd", precise: bool = False, kv_splits: int = 0,
                                 cu_seqlens_q: Optional[torch.Tensor] = None,
                                 max_seqlen_q: Optional[int] = None) -> int:
    """Workspace bytes attn_prefill_fwd uses for its tail split with these shapes on the
    current device (0: the call does not split)."""
    if cu_seqlens_q is not None:
        B, (_, Hq, d), Sq = cu_seqlens_q.numel() - 1, q.shape, int(max_seqlen_q)
    elif layout == "bshd":
        B, Sq, Hq, d = q.shape
    else:
        B, Hq, Sq, d = q.shape
    a = _lib.PrefillArgs(
        None, None, None, None, None, None, None, _ptr(cu_seqlens_q), B, Hq, int(num_heads_kv), Sq, int(seqlen_k),
        d, 0, 0, _DT[q.dtype], _DT[q.dtype], _LAYOUT[layout], int(bool(causal)), int(bool(precise)), 0.0, 0,
        int(kv_splits), None, 0)
    return int(_lib.load().attn_prefill_workspace_bytes(ctypes.byref(a)))


def attn_decode_workspace_bytes(batch: int, num_heads_q: int, num_splits: int, head_dim: int) -> int:
    return int(_lib.load().attn_decode_workspace_bytes(batch, num_heads_q, num_splits, head_dim))


def _decode_shapes(q, k_cache, v_cache, block_table, seqlens_k):
    """(B, Hq, Hkv, d, num_blocks) of a decode call, after checking that the tensors agree."""
    _need(q, "q", (torch.float16, torch.bfloat16))
    _need(k_cache, "k_cache", (q.dtype,))
    _need(v_cache, "v_cache", (q.dtype,))
    _need(block_table, "block_table", (torch.int32,))
    _need(seqlens_k, "seqlens_k", (torch.int32,))
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must be [num_blocks, 64, Hkv, d] of the same shape")
    num_blocks, page, Hkv, d = k_cache.shape
    if page != _lib.ATTN_PAGE_SIZE:
        raise ValueError(f"pages must hold {_lib.ATTN_PAGE_SIZE} tokens")
    if block_table.dim() != 2:
        raise ValueError("block_table must be [batch, max_blocks_per_seq]")
    B = block_table.shape[0]
    if seqlens_k.numel() != B:
        raise ValueError("seqlens_k must hold one length per sequence")
    if B and q.numel() % (B * d) != 0:
        raise ValueError("q must hold batch x num_heads_q x head_dim elements")
    Hq = q.numel() // (B * d) if B else 0
    return B, Hq, Hkv, d, num_blocks


def _decode_outputs(out, lse, B, Hq, d):
    _need(out, "out", tuple(_DT))
    if out.numel() != B * Hq * d:
        raise ValueError("out must hold batch x num_heads_q x head_dim elements")
    if lse is not None:
        _need(lse, "lse", (torch.float32,))
        if lse.numel() != B * Hq:
            raise ValueError("lse must hold batch x num_heads_q elements")


def attn_decode_fwd(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    block_table: torch.Tensor, seqlens_k: torch.Tensor, *, max_seqlen_k: int,
                    num_splits: int, out: Optional[torch.Tensor] = None,
                    out_dtype: Optional[torch.dtype] = None, lse: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, scale: float = 0.0,
                    out_round: str = "rtne", stream=None) -> torch.Tensor:
    """Split-KV decode. q: [B, Hq, d] (or any shape with B*Hq*d elements in that order)."""
    B, Hq, Hkv, d, num_blocks = _decode_shapes(q, k_cache, v_cache, block_table, seqlens_k)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype or q.dtype, device=q.device)
    _decode_outputs(out, lse, B, Hq, d)
    need = attn_decode_workspace_bytes(B, Hq, num_splits, d) if B else 0
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", (torch.uint8,))
    a = _lib.DecodeArgs(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seqlens_k), _ptr(out),
        _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
        B, Hq, Hkv, d, num_blocks, block_table.shape[1], int(max_seqlen_k), int(num_splits),
        _DT[q.dtype], _DT[out.dtype], float(scale), _round(out_round))
    _check(_lib.load().attn_decode_fwd(ctypes.byref(a), _stream(stream)))
    return out


def attn_decode_fwd_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            block_table: torch.Tensor, seqlens_k: torch.Tensor, *, max_seqlen_k: int,
                            num_splits: int, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                            scale: float = 0.0, out_round: str = "rtne", stream=None) -> torch.Tensor:
    """Split-KV decode without a workspace (the library's static device scratch).

    Same arguments as attn_decode_fwd, but ``out`` must be passed (this call allocates
    nothing, here or in the library). Calls that overlap on one device race on the
    shared scratch; calls ordered on one stream do not."""
    B, Hq, Hkv, d, num_blocks = _decode_shapes(q, k_cache, v_cache, block_table, seqlens_k)
    _decode_outputs(out, lse, B, Hq, d)
    a = _lib.DecodeArgs(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seqlens_k), _ptr(out),
        _ptr(lse), None, 0, B, Hq, Hkv, d, num_blocks, block_table.shape[1], int(max_seqlen_k),
        int(num_splits), _DT[q.dtype], _DT[out.dtype], float(scale), _round(out_round))
    _check(_lib.load().attn_decode_fwd_noalloc(ctypes.byref(a), _stream(stream)))
    return out


def attn_splitkv_combine(partial_o: torch.Tensor, partial_lse: torch.Tensor, *,
                         out: Optional[torch.Tensor] = None, out_dtype=torch.float32,
                         lse: Optional[torch.Tensor] = None, out_round: str = "rtne",
                         stream=None) -> torch.Tensor:
    """Merge partials: partial_o [B, H, S, d] fp32, partial_lse [B, H, S] fp32 -> [B, H, d]."""
    _need(partial_o, "partial_o", (torch.float32,))
    _need(partial_lse, "partial_lse", (torch.float32,))
    if partial_o.dim() != 4 or tuple(partial_lse.shape) != tuple(partial_o.shape[:3]):
        raise ValueError("partial_o must be [B, H, S, d] and partial_lse [B, H, S]")
    B, H, S, d = partial_o.shape
    if out is None:
        out = torch.empty((B, H, d), dtype=out_dtype, device=partial_o.device)
    _decode_outputs(out, lse, B, H, d)
    a = _lib.CombineArgs(_ptr(partial_o), _ptr(partial_lse), _ptr(out), _ptr(lse), B, H, S, d,
                         _DT[out.dtype], _round(out_round))
    _check(_lib.load().attn_splitkv_combine(ctypes.byref(a), _stream(stream)))
    return out


def attn_device_info(device: int = 0) -> dict:
    """Facts of HIP device ``device`` as the library reads them (attn_device_info)."""
    info = _lib.DeviceInfo()
    _check(_lib.load().attn_device_info(int(device), ctypes.byref(info)))
    return {f: (getattr(info, f).decode(errors="replace") if f in ("name", "arch") else int(getattr(info, f)))
            for f, _ in _lib.DeviceInfo._fields_}
