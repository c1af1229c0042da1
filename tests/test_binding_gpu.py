"""The Python binding refuses tensors whose shapes disagree before anything reaches the C
ABI (which sees only pointers and sizes, so a mismatched tensor there would be read out of
bounds). Device tensors are needed to reach these checks, hence a GPU test; no kernel runs."""
import pytest
import torch

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def _prefill_dense(**kw):
    from attention_forward_tiled_amd import attn_prefill_fwd
    args = dict(q=_t(2, 100, 8, 128), k=_t(2, 200, 2, 128), v=_t(2, 200, 2, 128))
    args.update(kw)
    return attn_prefill_fwd(args.pop("q"), args.pop("k"), args.pop("v"), causal=True, **args)


def _prefill_paged(**kw):
    from attention_forward_tiled_amd import attn_prefill_fwd
    args = dict(q=_t(2, 100, 8, 128), k=_t(8, 64, 2, 128), v=_t(8, 64, 2, 128),
                block_table=_i32(2, 4), seqlens_k=_i32(2, fill=200))
    args.update(kw)
    return attn_prefill_fwd(args.pop("q"), args.pop("k"), args.pop("v"), causal=True, **args)


def _i32(*shape, fill=0):
    return torch.full(shape, fill, dtype=torch.int32, device="cuda")


# (call, keyword overrides built on the device inside the test, expected message)
PREFILL_BAD = [
    (_prefill_dense, lambda: dict(v=_t(2, 201, 2, 128)), "same shape"),
    (_prefill_dense, lambda: dict(k=_t(2, 200, 2, 64), v=_t(2, 200, 2, 64)), "head size"),
    (_prefill_dense, lambda: dict(k=_t(1, 200, 2, 128), v=_t(1, 200, 2, 128)), "batch of q"),
    (_prefill_dense, lambda: dict(seqlens_k=_i32(3)), "one length per sequence"),
    (_prefill_paged, lambda: dict(block_table=_i32(3, 4)), "block_table"),
    (_prefill_dense, lambda: dict(out=_t(2, 100, 8, 64)), "shape of q"),
]


@pytest.mark.parametrize("fn,kw,msg", PREFILL_BAD, ids=[m for _, _, m in PREFILL_BAD])
def test_prefill_binding_rejects_mismatched_tensors(fn, kw, msg):
    with pytest.raises(ValueError, match=msg):
        fn(**kw())


def _decode(fn_name="attn_decode_fwd", **kw):
    import attention_forward_tiled_amd as A
    args = dict(q=_t(2, 8, 128), k_cache=_t(8, 64, 2, 128), v_cache=_t(8, 64, 2, 128),
                block_table=_i32(2, 4), seqlens_k=_i32(2, fill=200))
    if fn_name == "attn_decode_fwd_noalloc":
        args["out"] = _t(2, 8, 128)
    args.update(kw)
    return getattr(A, fn_name)(args.pop("q"), args.pop("k_cache"), args.pop("v_cache"),
                               args.pop("block_table"), args.pop("seqlens_k"), max_seqlen_k=200,
                               num_splits=4, **args)


DECODE_BAD = [
    (lambda: dict(v_cache=_t(8, 64, 2, 64)), "same shape"),
    (lambda: dict(seqlens_k=_i32(3)), "one length per sequence"),
    (lambda: dict(q=_t(2, 8, 100)), "batch x num_heads_q x head_dim"),
    (lambda: dict(out=_t(2, 8, 64)), "out must hold"),
    (lambda: dict(lse=torch.zeros((2, 4), device="cuda")), "lse must hold"),
    (lambda: dict(block_table=_i32(8)), "block_table"),
]


@pytest.mark.parametrize("fn_name", ["attn_decode_fwd", "attn_decode_fwd_noalloc"])
@pytest.mark.parametrize("kw,msg", DECODE_BAD, ids=[m for _, m in DECODE_BAD])
def test_decode_binding_rejects_mismatched_tensors(fn_name, kw, msg):
    with pytest.raises(ValueError, match=msg):
        _decode(fn_name, **kw())


def test_combine_binding_rejects_mismatched_tensors():
    from attention_forward_tiled_amd import attn_splitkv_combine
    po = torch.zeros((2, 4, 3, 128), device="cuda")
    with pytest.raises(ValueError, match="partial_lse"):
        attn_splitkv_combine(po, torch.zeros((2, 4, 2), device="cuda"))
    with pytest.raises(ValueError, match="out must hold"):
        attn_splitkv_combine(po, torch.zeros((2, 4, 3), device="cuda"), out=torch.zeros((2, 4, 64), device="cuda"))
