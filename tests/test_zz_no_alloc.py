"""The allocation-free decode (attn_decode_fwd_noalloc) against attn_decode_fwd.

Both entry points run the same kernels; the allocation-free one keeps the split
partials and the partition plan in the library's static device scratch instead of a
caller workspace. Two calls in a row, the second on a smaller input, so that what the
first call left in the scratch must not reach the second result; each is compared
with attn_decode_fwd on the same input (bit for bit: same kernels, same order) and
with the fp64 oracle within the decode tolerance.
"""
import numpy as np
import pytest
import torch

from attn_workloads import DecodeCase, make_decode_inputs
from gpu_util import TOL, dev, dev_i32, lse_tolerance, max_abs_err, oracle_decode, say, to_f64

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _run(fn, inp, splits, **kw):
    c = inp.case
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[c.dtype]
    out = torch.full((c.batch, c.heads_q, c.head_dim), float("nan"), dtype=tdt, device="cuda")
    lse = torch.full((c.batch, c.heads_q), float("nan"), dtype=torch.float32, device="cuda")
    fn(dev(inp.q, c.dtype), dev(inp.k_cache, c.dtype), dev(inp.v_cache, c.dtype),
       dev_i32(inp.block_table), dev_i32(inp.seqlens_k), max_seqlen_k=inp.max_seqlen_k,
       num_splits=splits, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("splits", [16, 1])
def test_noalloc_decode_matches_workspace_decode(splits):
    from attention_forward_tiled_amd import attn_decode_fwd, attn_decode_fwd_noalloc
    big = DecodeCase("noalloc_big", 8, 32, 8, 128, "bf16",
                     lengths_fixed=(30000, 1, 4097, 64, 12345, 65536, 700, 2000))
    small = DecodeCase("noalloc_small", 3, 8, 2, 64, "f16", lengths_fixed=(100, 5000, 63))
    for case, seed in ((big, 31), (small, 32)):
        say(f"decode without allocation, {case} num_splits={splits}")
        inp = make_decode_inputs(case, seed=seed)
        o_na, l_na = _run(attn_decode_fwd_noalloc, inp, splits)
        o_ws, l_ws = _run(attn_decode_fwd, inp, splits)
        assert bool(torch.isfinite(o_na).all()) and not bool(torch.isnan(l_na).any())
        assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16))
        assert torch.equal(l_na.view(torch.int32), l_ws.view(torch.int32))
        Oref, lref = oracle_decode(inp, per_call=1)
        err = max_abs_err(to_f64(o_na), Oref)
        say(f"  bit-equal to attn_decode_fwd; max abs err vs oracle {err:.3e}")
        assert err <= TOL[case.dtype]
        assert np.abs(to_f64(l_na) - lref).max() <= lse_tolerance(case.dtype)


def test_noalloc_decode_rejects_sizes_above_the_scratch():
    from attention_forward_tiled_amd import AttnError, attn_decode_fwd_noalloc
    case = DecodeCase("noalloc_too_big", 64, 64, 8, 128, "bf16", lengths_fixed=(64,) * 64)
    inp = make_decode_inputs(case, seed=33)
    say("decode without allocation, size above the scratch maximum")
    with pytest.raises(AttnError, match="maximum"):
        _run(attn_decode_fwd_noalloc, inp, 16)
