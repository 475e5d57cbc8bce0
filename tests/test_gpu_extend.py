"""Prefix-cached extend over a paged KV cache, with prefill, extend and decode
sequences mixed in one launch (RL-Kernel page, section 2: one arithmetic path
serves full-sequence forward, prefill, prefix-cached extend and single-token
paged decode).  Parity against the fp64 oracle on keys the oracle gathers from
the same pages, and bitwise identity: paged extend = contiguous prefill =
decode, split = monolithic, and a sequence's rows do not depend on the other
sequences of the launch.  Dead cache slots and spare pages hold NaN."""
import numpy as np
import pytest
import torch

import synth
from gpu_utils import (assert_bitwise, compare, dev, extend_workspace, note, oracle_extend,
                       run_decode, run_extend, run_prefill)

pytestmark = pytest.mark.gpu

MONO, SPLIT = 0, 1

# prefill (q = ctx), extend (q < ctx, prefixes across chunk boundaries) and
# decode (q = 1) sequences, ragged everywhere
MIX_CTX = [300, 1, 1100, 64, 2000, 513, 777]
MIX_Q = [300, 1, 37, 1, 700, 1, 777]


def _check_lse(lse, ref_lse):
    lg = lse.cpu().double().numpy()
    assert np.array_equal(np.isneginf(lg), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    if fin.any():
        assert np.abs(lg[fin] - ref_lse[fin]).max() < 2e-3


@pytest.mark.parametrize("schedule", [MONO, SPLIT])
@pytest.mark.parametrize("causal", [True, False])
def test_mixed_batch_parity(schedule, causal):
    inp = synth.extend_inputs(41, MIX_CTX, MIX_Q, 8, 2, 128, causal=causal)
    note(f"paged extend bf16 ctx={MIX_CTX} q={MIX_Q} causal={causal} schedule={schedule}")
    o, lse = run_extend(inp, schedule, return_lse=True)
    ref, ref_lse = oracle_extend(inp)
    compare(o, ref, False, label="O paged extend")
    _check_lse(lse, ref_lse)


@pytest.mark.parametrize("d,hq,hkv", [(64, 2, 1), (192, 4, 4)])
def test_mixed_batch_head_dims(d, hq, hkv):
    inp = synth.extend_inputs(43, [300, 1000, 1], [300, 77, 1], hq, hkv, d)
    note(f"paged extend bf16 d={d}")
    o = run_extend(inp, MONO)
    ref, _ = oracle_extend(inp)
    compare(o, ref, False, label=f"O paged extend d={d}")


@pytest.mark.parametrize("d", [128, 192])
def test_mixed_batch_fp8(d):
    inp = synth.extend_inputs(45, [700, 1300, 1], [700, 100, 1], 4, 4, d, dtype="fp8")
    note(f"paged extend fp8 d={d}")
    o = run_extend(inp, SPLIT)
    ref, _ = oracle_extend(inp)
    compare(o, ref, True, label=f"O paged extend fp8 d={d}")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp8", 192)])
def test_extend_equals_prefill_and_decode(dtype, d):
    """Row i of a paged extend equals row L_k - L_q + i of the contiguous causal
    prefill of the whole sequence, and its last row equals the decode token."""
    ctx = [1, 63, 64, 65, 512, 513, 1000, 1537]
    ql = [1, 20, 64, 1, 100, 1, 999, 512]
    hq, hkv = 8, 2
    inp = synth.extend_inputs(47, ctx, ql, hq, hkv, d, dtype=dtype, full_q=True)
    note(f"extend = prefill = decode {dtype} d={d}")
    o_ext, l_ext = run_extend(inp, MONO, return_lse=True)
    pre = synth.PrefillInputs(inp.q_full, inp.k, inp.v, inp.cu_full, inp.cu_full, ctx, ctx, hq,
                              hkv, d, inp.scale, True, dtype, inp.q_scale, inp.k_scale,
                              inp.v_scale, inp.seed)
    o_pre, l_pre = run_prefill(pre, MONO, return_lse=True)
    tail = torch.cat([torch.arange(int(inp.cu_full[b + 1]) - ql[b], int(inp.cu_full[b + 1]))
                      for b in range(len(ctx))])
    assert_bitwise(o_ext, o_pre[tail.to(o_pre.device)], "extend rows vs prefill rows")
    assert_bitwise(l_ext, l_pre[tail.to(l_pre.device)], "extend lse vs prefill lse")
    # the decode token of every sequence: the last query row, through the decode kernel
    last = inp.cu_full[1:].long() - 1
    dec = synth.DecodeInputs(inp.q_full[last].contiguous(), inp.k_cache, inp.v_cache,
                             inp.page_table, inp.context_lens, hq, hkv, d, inp.page_size,
                             inp.scale, inp.seed, dtype, inp.q_scale, inp.k_scale, inp.v_scale)
    o_dec, l_dec = run_decode(dec, SPLIT, return_lse=True)
    ext_last = inp.cu_seqlens_q[1:].long() - 1
    assert_bitwise(o_dec, o_ext[ext_last.to(o_ext.device)], "decode vs extend last row")
    assert_bitwise(l_dec, l_ext[ext_last.to(l_ext.device)], "decode lse vs extend last row")


# Single-token rows of kv groups larger than one tile: a group packs into one
# tile set of several tiles (256 rows for bf16 up to D = 128, 128 for bf16
# D = 192 on four waves and for e4m3 D = 192), computed by the workgroups of
# the set's heads.
@pytest.mark.parametrize("dtype,d,hq", [("bf16", 128, 512), ("bf16", 192, 256),
                                        ("fp8", 192, 256)])
def test_groups_larger_than_a_tile(dtype, d, hq):
    ctx, ql = [3000, 700, 1, 1500], [1, 5, 1, 1]
    inp = synth.extend_inputs(47, ctx, ql, hq, 1, d, dtype=dtype)
    note(f"paged extend {dtype} d={d} group={hq} ctx={ctx} q={ql}")
    o, lse = run_extend(inp, MONO, return_lse=True)
    ref, ref_lse = oracle_extend(inp)
    compare(o, ref, dtype == "fp8", label=f"O group {hq}")
    _check_lse(lse, ref_lse)
    o_s, lse_s = run_extend(inp, SPLIT, return_lse=True)
    assert_bitwise(o_s, o, "O split vs monolithic")
    assert_bitwise(lse_s, lse, "lse split vs monolithic")
    o_w, lse_w = run_extend(inp, MONO, return_lse=True, workspace=extend_workspace(inp))
    assert_bitwise(o_w, o, "O with workspace vs without")
    assert_bitwise(lse_w, lse, "lse with workspace vs without")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_extend_split_equals_monolithic(dtype):
    inp = synth.extend_inputs(49, MIX_CTX, MIX_Q, 4, 2, 128, dtype=dtype)
    o1, l1 = run_extend(inp, MONO, return_lse=True)
    o2, l2 = run_extend(inp, SPLIT, return_lse=True)
    assert_bitwise(o1, o2, "paged extend O split vs monolithic")
    assert_bitwise(l1, l2, "paged extend lse split vs monolithic")


def test_mixed_batch_composition():
    """Each sequence of a mixed launch gives the same bits alone."""
    inp = synth.extend_inputs(51, MIX_CTX, MIX_Q, 4, 2, 128)
    o_all = run_extend(inp, MONO)
    for b in (0, 2, 3, 4):
        one = synth.ExtendInputs(
            inp.q[int(inp.cu_seqlens_q[b]):int(inp.cu_seqlens_q[b + 1])].contiguous(),
            synth.cu_seqlens([MIX_Q[b]]), inp.q_full, inp.k, inp.v, inp.cu_full, inp.k_cache,
            inp.v_cache, inp.page_table[b:b + 1].contiguous(), inp.context_lens[b:b + 1].clone(),
            [MIX_Q[b]], [MIX_CTX[b]], inp.hq, inp.hkv, inp.d, inp.page_size, inp.scale,
            inp.causal, inp.dtype)
        o_one = run_extend(one, MONO)
        r0, r1 = int(inp.cu_seqlens_q[b]), int(inp.cu_seqlens_q[b + 1])
        assert_bitwise(o_one, o_all[r0:r1], f"sequence {b} alone vs in the mixed batch")


def test_extend_sentinel_outside_valid_rows():
    """Rows of O outside [0, total_q) of the call survive a pre-fill (the
    epilogue's descriptor bound), and the valid rows are overwritten."""
    inp = synth.extend_inputs(53, [300, 1000], [300, 77], 4, 2, 128)
    tq = sum(inp.q_lens)
    big = torch.full((tq + 300, inp.hq, inp.d), 7.0, dtype=torch.bfloat16, device="cuda")
    view = big[:tq]
    run_extend(inp, MONO, out=view)
    assert torch.all(big[tq:] == 7.0), "rows past the call's rows were written"
    assert not torch.any(view == 7.0), "a valid row was not written"


def test_full_mixed_workload():
    """The benchmark's mixed batch at full size: prefill, extend and decode
    sequences in one launch, monolithic and split + merge (bit for bit the
    same), against the oracle on every element."""
    cfg = synth.MIXED_EXTEND
    inp = synth.extend_inputs(0, cfg["ctx_lens"], cfg["q_lens"], cfg["hq"], cfg["hkv"], cfg["d"],
                              spare_pages=cfg["spare_pages"])
    note("full mixed paged-extend workload")
    o = run_extend(inp, MONO)
    o_split = run_extend(inp, SPLIT)
    assert_bitwise(o_split, o, "mixed workload split vs monolithic")
    o_ws = run_extend(inp, MONO, workspace=extend_workspace(inp))
    assert_bitwise(o_ws, o, "mixed workload with the chunk-spread workspace vs without")
    note("oracle on every row")
    ref, _ = oracle_extend(inp)
    compare(o, ref, False, label=f"O full mixed extend (all {ref.size} elements)")
