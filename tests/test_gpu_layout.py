"""Paged-cache layouts: the kernels take page, token and head strides, so a
cache stored heads-outer ("HND", [num_pages, Hkv, 16, D]) gives the same bits as
the tokens-outer layout ("NHD", [num_pages, 16, Hkv, D]) whose parity with the
fp64 oracle the other tests establish."""
import pytest
import torch

import synth
from gpu_utils import assert_bitwise, dev, note

pytestmark = pytest.mark.gpu

MONO, SPLIT = 0, 1


def _hnd(t: torch.Tensor) -> torch.Tensor:
    return t.permute(0, 2, 1, 3).contiguous()


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp8", 192), ("fp8", 128)])
@pytest.mark.parametrize("schedule", [SPLIT, MONO])
def test_decode_layouts_bitwise(dtype, d, schedule):
    import deterministic_flash_attention_amd as dfa
    inp = synth.decode_inputs(81, 6, 8, 2, d, context_lens=[1, 17, 600, 1025, 3000, 5000],
                              spare_pages=8, dtype=dtype)
    note(f"decode layouts {dtype} d={d} schedule={schedule}")
    args = dict(softmax_scale=inp.scale, schedule=schedule,
                descales=(inp.q_scale, inp.k_scale, inp.v_scale), return_lse=True)
    q, pt, cl = dev(inp.q), dev(inp.page_table), dev(inp.context_lens)
    o1, l1 = dfa.decode(q, dev(inp.k_cache), dev(inp.v_cache), pt, cl, 5000, **args)
    o2, l2 = dfa.decode(q, dev(_hnd(inp.k_cache)), dev(_hnd(inp.v_cache)), pt, cl, 5000,
                        kv_layout="HND", **args)
    torch.cuda.synchronize()
    assert_bitwise(o1, o2, "decode O, HND vs NHD")
    assert_bitwise(l1, l2, "decode lse, HND vs NHD")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp8", 192)])
def test_extend_layouts_bitwise(dtype, d):
    import deterministic_flash_attention_amd as dfa
    ctx, ql = [300, 1, 1100, 2000], [300, 1, 37, 700]
    inp = synth.extend_inputs(83, ctx, ql, 8, 2, d, dtype=dtype)
    note(f"extend layouts {dtype} d={d}")
    args = dict(softmax_scale=inp.scale, descales=(inp.q_scale, inp.k_scale, inp.v_scale),
                return_lse=True)
    q, cq, pt, cl = dev(inp.q), dev(inp.cu_seqlens_q), dev(inp.page_table), dev(inp.context_lens)
    for sched in (MONO, SPLIT):
        o1, l1 = dfa.paged_extend(q, cq, dev(inp.k_cache), dev(inp.v_cache), pt, cl, max(ql),
                                  max(ctx), True, schedule=sched, **args)
        o2, l2 = dfa.paged_extend(q, cq, dev(_hnd(inp.k_cache)), dev(_hnd(inp.v_cache)), pt, cl,
                                  max(ql), max(ctx), True, schedule=sched, kv_layout="HND", **args)
        torch.cuda.synchronize()
        assert_bitwise(o1, o2, f"extend O (schedule {sched}), HND vs NHD")
        assert_bitwise(l1, l2, f"extend lse (schedule {sched}), HND vs NHD")
