"""Chunk spread of the monolithic paged extend (RL-Kernel page, section 2: a
mixed batch of prefill, extend and decode sequences goes through one launch).
Given a workspace, a single-token sequence whose context spans several chunks
has its chunks computed by otherwise idle workgroups of the same launch, and
the last of them folds the chunk partials.  Its rows must keep the bits of the
launch without a workspace (which the extend tests tie to prefill, decode and
the oracle), call after call, with the workspace's counters back at zero."""
import pytest
import torch

import synth
from gpu_utils import assert_bitwise, compare, extend_workspace, note, oracle_extend, run_extend

pytestmark = pytest.mark.gpu

MONO = 0

# Decode rows of 1 to 10 chunks next to prefill, extend and short decode rows.
CTX = [300, 5000, 1100, 64, 2000, 3000, 777, 1, 4097]
QL = [300, 1, 37, 1, 700, 1, 777, 1, 1]
LONG = 1  # the 5000-token decode row: 10 chunks


COUNTER_WORDS = 65536  # the counter region that opens the workspace


def _regions(ws, inp):
    """(ml [cmax, batch, hq, 2], counter region) views of the workspace."""
    import deterministic_flash_attention_amd as dfa
    b, cmax = len(inp.q_lens), dfa.attn_num_chunks(max(inp.ctx_lens))
    cells = cmax * b * inp.hq
    part = ws[COUNTER_WORDS:]
    ml = part[cells * inp.d:cells * (inp.d + 2)].view(cmax, b, inp.hq, 2)
    cnt = ws[:COUNTER_WORDS].view(torch.int32)
    return ml, cnt


def _spread_vs_single(inp, window=(-1, -1), calls=2):
    o_ref, l_ref = run_extend(inp, MONO, return_lse=True, window=window)
    ws = extend_workspace(inp)
    for call in range(calls):
        o, lse = run_extend(inp, MONO, return_lse=True, workspace=ws, window=window)
        assert_bitwise(o, o_ref, f"O with workspace (call {call}) vs without")
        assert_bitwise(lse, l_ref, f"lse with workspace (call {call}) vs without")
        _, cnt = _regions(ws, inp)
        assert int(torch.count_nonzero(cnt)) == 0, "counters not back at zero"
    return o_ref, ws


# bf16 spread tiles run a loop of their own: three K/V stages while the kv
# group's query heads fit below the third stage (96 rows at D = 128, 64 at
# D = 64), two beyond; groups of 64 (two computing waves), 128 and, at D = 64,
# 96 take the other paths.
@pytest.mark.parametrize("dtype,d,hq,hkv", [("bf16", 128, 8, 2), ("bf16", 64, 4, 1),
                                            ("bf16", 128, 4, 4), ("fp8", 128, 4, 2),
                                            ("fp8", 192, 4, 4), ("bf16", 128, 64, 1),
                                            ("bf16", 128, 128, 1), ("bf16", 64, 96, 1)])
def test_spread_equals_single_tile(dtype, d, hq, hkv):
    inp = synth.extend_inputs(61, CTX, QL, hq, hkv, d, dtype=dtype)
    note(f"chunk spread {dtype} d={d} hq={hq} hkv={hkv} ctx={CTX} q={QL}")
    _, ws = _spread_vs_single(inp)
    # The spread ran: every chunk partial of the long decode row's heads is in
    # the workspace (m finite, l >= 1), and no chunk past its context is.
    ml, _ = _regions(ws, inp)
    nch = (CTX[LONG] + 511) // 512
    m, l = ml[:nch, LONG, :, 0], ml[:nch, LONG, :, 1]
    assert torch.isfinite(m).all() and (l >= 1.0).all()
    assert int(torch.count_nonzero(ml[nch:, LONG])) == 0


@pytest.mark.parametrize("hq", [64, 128])
def test_spread_large_groups_against_oracle(hq):
    """Single-token rows of kv groups of 64 and 128 query heads (three and
    two K/V stages in the spread tile), against the oracle."""
    inp = synth.extend_inputs(67, CTX, QL, hq, 1, 128)
    o, _ = _spread_vs_single(inp, calls=1)
    cq = inp.cu_seqlens_q.tolist()
    rows = [cq[b] for b, q in enumerate(QL) if q == 1]
    ref = oracle_extend(inp, rows=rows)[0]
    compare(o, ref, False, rows=rows, label=f"O single-token rows, group {hq}, chunk spread")


def test_spread_against_oracle():
    inp = synth.extend_inputs(63, CTX, QL, 8, 2, 128)
    o, _ = _spread_vs_single(inp, calls=1)
    ref, _ = oracle_extend(inp)
    compare(o, ref, False, label="O paged extend with chunk spread")


def test_spread_with_left_window():
    """Decode rows whose window starts inside a chunk: the spread covers the
    chunks from the window's first one."""
    inp = synth.extend_inputs(65, CTX, QL, 8, 2, 128)
    _spread_vs_single(inp, window=(1500, -1))


def test_spread_decode_only_batch():
    """max_seqlen_q = 1: the launch's tile slots are widened so that every
    decode row has a slot per chunk."""
    ctx = [1, 700, 4097, 9000, 513]
    inp = synth.extend_inputs(67, ctx, [1] * len(ctx), 32, 8, 128)
    _spread_vs_single(inp)


def test_no_spread_for_bf16_d192():
    """bf16 D = 192 runs the single tile with or without a workspace, which
    then stays untouched."""
    inp = synth.extend_inputs(69, CTX, QL, 4, 4, 192)
    o_ref = run_extend(inp, MONO)
    ws = extend_workspace(inp)
    o = run_extend(inp, MONO, workspace=ws)
    assert_bitwise(o, o_ref, "bf16 D=192 with workspace vs without")
    assert int(torch.count_nonzero(ws)) == 0


def test_workspace_reused_across_batches():
    """One zero-filled workspace, sized for the largest call, serves launches of
    different batch shapes in turn (each call's partials land where another
    call's counters would be if the counters moved with the shape)."""
    import deterministic_flash_attention_amd as dfa
    batches = [(CTX, QL, 8, 2), ([9000, 1, 700], [1, 1, 700], 8, 2), (CTX[:4], QL[:4], 8, 4)]
    inps = [synth.extend_inputs(71 + i, c, q, hq, hkv, 128) for i, (c, q, hq, hkv) in
            enumerate(batches)]
    nbytes = max(dfa.attn_extend_workspace_bytes(len(i.q_lens), i.hq, i.hkv,
                                                 dfa.attn_num_chunks(max(i.ctx_lens)), i.d)
                 for i in inps)
    ws = torch.zeros((nbytes + 3) // 4, dtype=torch.float32, device="cuda")
    for rnd in range(2):
        for i, inp in enumerate(inps):
            o_ref = run_extend(inp, MONO)
            o = run_extend(inp, MONO, workspace=ws)
            assert_bitwise(o, o_ref, f"batch {i} round {rnd} with a shared workspace")
            assert int(torch.count_nonzero(ws[:COUNTER_WORDS])) == 0
