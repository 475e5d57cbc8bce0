"""Sliding-window (local) attention on the GPU: a left/right window on the
bottom-right diagonal, bounded in the kernels by the block ranges, the masks
and window-sized K/V descriptors (aiter MQA-logits page: num_records is the
window test).  Parity against the fp64 oracle's windowed mask, the closed form
of a zero left window, and the bitwise invariances with windows (split =
monolithic, decode = last prefill row, paged extend = prefill)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_utils import (assert_bitwise, compare, dev, note, oracle_inputs_prefill, run_decode,
                       run_prefill)

pytestmark = pytest.mark.gpu

MONO, SPLIT = 0, 1


def _prefill(inp, schedule, window, **kw):
    import deterministic_flash_attention_amd as dfa
    res = dfa.prefill(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.cu_seqlens_q),
                      dev(inp.cu_seqlens_k), max(inp.seqlens_q), max(inp.seqlens_k), inp.causal,
                      softmax_scale=inp.scale, schedule=schedule,
                      descales=(inp.q_scale, inp.k_scale, inp.v_scale), window=window, **kw)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("schedule", [MONO, SPLIT])
@pytest.mark.parametrize("case", [
    # (seqlens_q, seqlens_k, causal, window)
    ([1100, 1, 600], None, True, (100, -1)),
    ([1100, 1, 600], None, True, (513, -1)),     # window edge inside a later chunk
    ([900], None, False, (64, 200)),             # two-sided, not causal
    ([900], None, False, (-1, 70)),              # right window only
    ([100, 37], [700, 1300], True, (300, -1)),   # extend rows with a window
])
def test_window_parity(schedule, case):
    sq, sk, causal, win = case
    inp = synth.prefill_inputs(61, sq, 8, 2, 128, causal, seqlens_k=sk)
    note(f"window {win} q={sq} k={sk} causal={causal} schedule={schedule}")
    o, lse = _prefill(inp, schedule, win, return_lse=True)
    q, k, v = oracle_inputs_prefill(inp)
    ref, ref_lse = oracle.attention(q, k, v, inp.cu_seqlens_q.numpy(), inp.cu_seqlens_k.numpy(),
                                    8, 2, inp.scale, causal, window=win)
    compare(o, ref, False, label=f"O window {win}")
    lg = lse.cpu().double().numpy()
    assert np.array_equal(np.isneginf(lg), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    assert np.abs(lg[fin] - ref_lse[fin]).max() < 2e-3


@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (192, "bf16"), (192, "fp8")])
def test_window_head_dims(d, dtype):
    inp = synth.prefill_inputs(63, [700, 300], 4, 4, d, True, dtype=dtype)
    note(f"window d={d} {dtype}")
    o = _prefill(inp, SPLIT if dtype == "fp8" else MONO, (200, -1))
    q, k, v = oracle_inputs_prefill(inp)
    ref, _ = oracle.attention(q, k, v, inp.cu_seqlens_q.numpy(), inp.cu_seqlens_k.numpy(), 4, 4,
                              inp.scale, True, window=(200, -1))
    compare(o, ref, dtype == "fp8", label=f"O window d={d} {dtype}")


@pytest.mark.parametrize("schedule", [MONO, SPLIT])
def test_zero_left_window_is_the_diagonal_value_row(schedule):
    """With a left window of 0 under the causal mask a row sees only its own key:
    O_i is V[i + L_k - L_q] bit for bit (p is exp2 of a rounding residual, so
    P = 1 in bf16 and O = V / L rounds back to V)."""
    sq, sk = [300, 77], [300, 500]
    inp = synth.prefill_inputs(65, sq, 4, 2, 128, True, seqlens_k=sk)
    o = _prefill(inp, schedule, (0, -1))
    rows, keys = [], []
    for b in range(2):
        for i in range(sq[b]):
            rows.append(int(inp.cu_seqlens_q[b]) + i)
            keys.append(int(inp.cu_seqlens_k[b]) + i + sk[b] - sq[b])
    v_diag = inp.v[keys].repeat_interleave(2, dim=1)  # kv head g serves q heads 2g, 2g+1
    assert_bitwise(o[rows].cpu(), v_diag, "O vs its diagonal V row")


@pytest.mark.parametrize("case", [
    ([1100, 1, 600], None, True, (100, -1)),
    ([900], None, False, (64, 200)),
    ([100, 37], [700, 1300], True, (300, -1)),
])
def test_window_split_equals_monolithic(case):
    sq, sk, causal, win = case
    inp = synth.prefill_inputs(67, sq, 4, 2, 128, causal, seqlens_k=sk)
    o1, l1 = _prefill(inp, MONO, win, return_lse=True)
    o2, l2 = _prefill(inp, SPLIT, win, return_lse=True)
    assert_bitwise(o1, o2, f"window {win} O split vs monolithic")
    assert_bitwise(l1, l2, f"window {win} lse split vs monolithic")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp8", 192)])
@pytest.mark.parametrize("wl", [0, 100, 511, 512, 2000])
def test_window_decode_equals_last_prefill_row(dtype, d, wl):
    lens = [1, 64, 65, 513, 1000, 1537, 3000]
    hq, hkv = 8, 2
    inp = synth.prefill_inputs(69, lens, hq, hkv, d, True, dtype=dtype)
    note(f"window decode = prefill {dtype} d={d} wl={wl}")
    o_pre = _prefill(inp, MONO, (wl, -1))
    # the same keys laid out as pages
    ps, pages, rows = 16, [], []
    table = torch.zeros(len(lens), (max(lens) + ps - 1) // ps, dtype=torch.int32)
    npg = 0
    for b, n in enumerate(lens):
        k0 = int(inp.cu_seqlens_k[b])
        for pgi in range((n + ps - 1) // ps):
            blk = torch.zeros(ps, hkv, d, dtype=inp.k.dtype), torch.zeros(ps, hkv, d, dtype=inp.v.dtype)
            t0, t1 = pgi * ps, min(n, pgi * ps + ps)
            blk[0][:t1 - t0] = inp.k[k0 + t0:k0 + t1]
            blk[1][:t1 - t0] = inp.v[k0 + t0:k0 + t1]
            pages.append(blk)
            table[b, pgi] = npg
            npg += 1
        rows.append(int(inp.cu_seqlens_q[b + 1]) - 1)
    kc = torch.stack([p[0] for p in pages]).contiguous()
    vc = torch.stack([p[1] for p in pages]).contiguous()
    dec = synth.DecodeInputs(inp.q[rows].contiguous(), kc, vc, table,
                             torch.tensor(lens, dtype=torch.int32), hq, hkv, d, ps, inp.scale,
                             inp.seed, dtype, inp.q_scale, inp.k_scale, inp.v_scale)
    import deterministic_flash_attention_amd as dfa
    for sched in (SPLIT, MONO):
        o_dec = dfa.decode(dev(dec.q), dev(kc), dev(vc), dev(table), dev(dec.context_lens),
                           max(lens), softmax_scale=inp.scale, schedule=sched,
                           descales=(inp.q_scale, inp.k_scale, inp.v_scale), window_left=wl)
        torch.cuda.synchronize()
        assert_bitwise(o_dec, o_pre[rows], f"decode (schedule {sched}) vs last prefill row")


def test_window_paged_extend_equals_prefill():
    ctx = [1, 300, 1100, 2000]
    ql = [1, 300, 37, 700]
    inp = synth.extend_inputs(71, ctx, ql, 8, 2, 128, full_q=True)
    import deterministic_flash_attention_amd as dfa
    win = (250, -1)
    o_ext = dfa.paged_extend(dev(inp.q), dev(inp.cu_seqlens_q), dev(inp.k_cache),
                             dev(inp.v_cache), dev(inp.page_table), dev(inp.context_lens),
                             max(ql), max(ctx), True, softmax_scale=inp.scale, window=win)
    pre = synth.PrefillInputs(inp.q_full, inp.k, inp.v, inp.cu_full, inp.cu_full, ctx, ctx, 8, 2,
                              128, inp.scale, True, "bf16", seed=inp.seed)
    o_pre = _prefill(pre, MONO, win)
    tail = torch.cat([torch.arange(int(inp.cu_full[b + 1]) - ql[b], int(inp.cu_full[b + 1]))
                      for b in range(len(ctx))])
    assert_bitwise(o_ext, o_pre[tail.to(o_pre.device)], "windowed extend rows vs prefill rows")


def test_full_dense_sliding_window():
    """The dense workload's shape with a causal 1024-key sliding window,
    monolithic and split + merge (bit for bit the same), against the oracle on
    every element."""
    cfg = synth.DENSE_PREFILL
    inp = synth.prefill_inputs(0, cfg["seqlens"], cfg["hq"], cfg["hkv"], cfg["d"], True)
    note("full dense causal sliding window 1024")
    o = _prefill(inp, MONO, (1024, -1))
    o_split = _prefill(inp, SPLIT, (1024, -1))
    assert_bitwise(o_split, o, "sliding window split vs monolithic")
    note("oracle on every row")
    q, k, v = oracle_inputs_prefill(inp)
    ref, _ = oracle.attention(q, k, v, inp.cu_seqlens_q.numpy(), inp.cu_seqlens_k.numpy(),
                              cfg["hq"], cfg["hkv"], inp.scale, True, window=(1024, -1))
    compare(o, ref, False, label=f"O dense sliding window (all {ref.size} elements)")
