"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, element by element, at the stated tolerances
(bf16: max_abs <= 1e-2 and mean_abs <= 1e-3; fp8: max_abs <= 6e-2 against the
oracle on the dequantised inputs)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_utils import (assert_bitwise, compare, dev, note, oracle_inputs_prefill, run_decode,
                       run_prefill)

pytestmark = pytest.mark.gpu

MONO, SPLIT = 0, 1


def _prefill_case(seqlens_q, seqlens_k, hq, hkv, d, causal, dtype, seed, schedule, rows=None):
    inp = synth.prefill_inputs(seed, seqlens_q, hq, hkv, d, causal, seqlens_k=seqlens_k,
                               dtype=dtype)
    note(f"prefill {dtype} q={seqlens_q} k={seqlens_k} hq={hq} hkv={hkv} d={d} causal={causal} "
         f"seed={seed} schedule={schedule}")
    o, lse = run_prefill(inp, schedule, return_lse=True)
    q, k, v = oracle_inputs_prefill(inp)
    ref, ref_lse = oracle.attention(q, k, v, inp.cu_seqlens_q.numpy(), inp.cu_seqlens_k.numpy(),
                                    hq, hkv, inp.scale, causal, rows=rows)
    compare(o, ref, dtype == "fp8", rows=rows, label="O")
    lg = lse.cpu().double().numpy()
    lr = ref_lse if rows is None else ref_lse[rows]
    lg = lg if rows is None else lg[rows]
    assert np.array_equal(np.isneginf(lg), np.isneginf(lr))
    fin = np.isfinite(lr)
    if fin.any():
        assert np.abs(lg[fin] - lr[fin]).max() < 2e-3
    return inp, o


@pytest.mark.parametrize("schedule", [MONO, SPLIT])
def test_tiny_causal_gqa(schedule):
    # 300 rows: not a multiple of 64 or 128, three 128-row tiles with 84 padded rows
    for seed in range(3):
        _prefill_case([300], None, 2, 1, 64, True, "bf16", seed, schedule)


@pytest.mark.parametrize("schedule", [MONO, SPLIT])
def test_dense_ragged_multi_chunk(schedule):
    _prefill_case([1100], None, 4, 4, 128, False, "bf16", 7, schedule)


@pytest.mark.parametrize("schedule", [MONO, SPLIT])
def test_causal_gqa_varlen_small(schedule):
    _prefill_case([600, 250, 1, 397], None, 8, 2, 128, True, "bf16", 3, schedule)


@pytest.mark.parametrize("schedule", [MONO, SPLIT])
def test_extend_bottom_right(schedule):
    # prefix-cached extend: fewer queries than keys, causal aligned bottom-right
    _prefill_case([100, 1, 37], [700, 513, 64], 4, 2, 128, True, "bf16", 5, schedule)


def test_more_queries_than_keys_all_masked_rows():
    inp, o = _prefill_case([200], [70], 2, 1, 64, True, "bf16", 9, MONO)
    assert torch.all(o[:130].float() == 0)


def test_empty_and_zero_key_sequences():
    _prefill_case([0, 130, 5], [0, 130, 0], 2, 2, 64, False, "bf16", 11, MONO)
    _prefill_case([0, 130, 5], [0, 130, 0], 2, 2, 64, False, "bf16", 11, SPLIT)


def test_head_dim_192_bf16():
    _prefill_case([333], None, 2, 1, 192, True, "bf16", 13, MONO)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("schedule", [MONO, SPLIT])
def test_fp8_wide_head_small(causal, schedule):
    _prefill_case([700], None, 4, 4, 192, causal, "fp8", 17, schedule)


def test_fp8_head_dim_128():
    _prefill_case([300, 129], None, 4, 2, 128, True, "fp8", 19, MONO)


# ---------------------------------------------------------------- decode
def _decode_case(ctx, hq, hkv, d, seed, schedule, dtype="bf16", spare=16):
    inp = synth.decode_inputs(seed, len(ctx), hq, hkv, d, context_lens=ctx, spare_pages=spare,
                              dtype=dtype)
    note(f"decode {dtype} ctx={ctx[:8]}.. hq={hq} hkv={hkv} d={d} seed={seed} sched={schedule}")
    o, lse = run_decode(inp, schedule, return_lse=True)
    if dtype == "fp8":
        q = oracle.dequantize_e4m3(inp.q.numpy(), inp.q_scale)
        kc = oracle.dequantize_e4m3(inp.k_cache.numpy(), inp.k_scale)
        vc = oracle.dequantize_e4m3(inp.v_cache.numpy(), inp.v_scale)
    else:
        q, kc, vc = synth.to_f64(inp.q), inp.k_cache.float().numpy(), inp.v_cache.float().numpy()
    ref, ref_lse = oracle.paged_decode(q, kc, vc, inp.page_table.numpy(), inp.context_lens.numpy(),
                                       hq, hkv, inp.scale, inp.page_size)
    compare(o, ref, dtype == "fp8", label="decode O")
    lg = lse.cpu().double().numpy()
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isneginf(lg), np.isneginf(ref_lse))
    if fin.any():
        assert np.abs(lg[fin] - ref_lse[fin]).max() < 2e-3
    return inp, o


CTX_SMALL = [1, 15, 16, 17, 63, 64, 65, 511, 512, 513, 1500, 2047]


@pytest.mark.parametrize("schedule", [SPLIT, MONO])
def test_decode_small(schedule):
    _decode_case(CTX_SMALL, 32, 8, 128, 21, schedule)


def test_decode_gqa_group_2_head_dim_64():
    _decode_case([5, 700, 1025], 4, 2, 64, 23, SPLIT)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (16, 2), (32, 1)])
def test_decode_group_sizes(hq, hkv, dtype):
    """One, eight and 32 query heads per kv head (32: every column of the MFMA
    tile is a query and none reads the zero row), against the oracle, with the
    two schedules equal bit for bit."""
    ctx = [1, 64, 513, 1100]
    _, o_split = _decode_case(ctx, hq, hkv, 128, 29, SPLIT, dtype=dtype)
    _, o_mono = _decode_case(ctx, hq, hkv, 128, 29, MONO, dtype=dtype)
    assert torch.equal(o_split.view(torch.int16), o_mono.view(torch.int16)), "split != monolithic"


def test_decode_fp8():
    _decode_case([3, 600, 1700], 8, 2, 128, 25, SPLIT, dtype="fp8")


def test_decode_zero_context():
    inp, o = _decode_case([0, 40], 4, 1, 128, 27, SPLIT)
    assert torch.all(o[0].float() == 0)


# ------------------------------------- full-size workloads, every element
# Each workload at its full size, in both schedules (split = the split kernel
# plus attn_chunk_merge), against the oracle on every row, head and column;
# max_abs and mean_abs are taken over all elements.  The schedules must also
# agree bit for bit.
def _full_prefill(cfg, causal, dtype):
    inp = synth.prefill_inputs(0, cfg["seqlens"], cfg["hq"], cfg["hkv"], cfg["d"], causal,
                               dtype=dtype)
    note(f"full {cfg['name']} {dtype} causal={causal}: GPU monolithic and split")
    o_mono, lse_mono = run_prefill(inp, MONO, return_lse=True)
    o_split, lse_split = run_prefill(inp, SPLIT, return_lse=True)
    assert_bitwise(o_split, o_mono, "O split vs monolithic")
    assert_bitwise(lse_split, lse_mono, "lse split vs monolithic")
    note("oracle on every row")
    q, k, v = oracle_inputs_prefill(inp)
    ref, ref_lse = oracle.attention(q, k, v, inp.cu_seqlens_q.numpy(), inp.cu_seqlens_k.numpy(),
                                    cfg["hq"], cfg["hkv"], inp.scale, causal)
    for name, o, lse in (("monolithic", o_mono, lse_mono), ("split", o_split, lse_split)):
        compare(o, ref, dtype == "fp8", label=f"O {name} (all {ref.size} elements)")
        lg = lse.cpu().double().numpy()
        assert np.array_equal(np.isneginf(lg), np.isneginf(ref_lse))
        fin = np.isfinite(ref_lse)
        assert np.abs(lg[fin] - ref_lse[fin]).max() < 2e-3


def test_full_dense_prefill():
    _full_prefill(synth.DENSE_PREFILL, False, "bf16")


def test_full_causal_varlen():
    _full_prefill(synth.CAUSAL_VARLEN, True, "bf16")


@pytest.mark.parametrize("causal", [False, True])
def test_full_fp8_wide_head(causal):
    _full_prefill(dict(synth.FP8_WIDE, causal=causal), causal, "fp8")


def test_full_tiny_causal_gqa():
    _full_prefill(synth.TINY_CAUSAL, True, "bf16")


def test_full_paged_decode_every_sequence():
    """All 64 sequences of the paged decode workload, split + merge and
    monolithic, over the tokens-outer ("NHD") cache and the heads-outer ("HND")
    cache the benchmark times, each against the oracle on every element;
    dead slots and spare pages hold NaN."""
    import deterministic_flash_attention_amd as dfa
    cfg = synth.PAGED_DECODE
    inp = synth.decode_inputs(0, cfg["batch"], cfg["hq"], cfg["hkv"], cfg["d"],
                              ctx_min=cfg["ctx_min"], ctx_max=cfg["ctx_max"],
                              spare_pages=cfg["spare_pages"])
    mc = int(inp.context_lens.max())
    note(f"full decode: sum ctx = {int(inp.context_lens.sum())}, max ctx = {mc}")
    outs = {}
    for layout in ("NHD", "HND"):
        kc, vc = inp.k_cache, inp.v_cache
        if layout == "HND":
            kc, vc = kc.permute(0, 2, 1, 3), vc.permute(0, 2, 1, 3)
        kc, vc = dev(kc), dev(vc)
        for sched in (SPLIT, MONO):
            o, lse = dfa.decode(dev(inp.q), kc, vc, dev(inp.page_table), dev(inp.context_lens), mc,
                                softmax_scale=inp.scale, schedule=sched, return_lse=True,
                                kv_layout=layout)
            torch.cuda.synchronize()
            outs[(layout, sched)] = (o, lse)
        del kc, vc
    o_ref, lse_ref = outs[("NHD", SPLIT)]
    for key, (o, lse) in outs.items():
        assert_bitwise(o, o_ref, f"decode O {key} vs NHD split")
        assert_bitwise(lse, lse_ref, f"decode lse {key} vs NHD split")
    note("oracle on every sequence")
    ref, ref_lse = oracle.paged_decode(synth.to_f64(inp.q), inp.k_cache.float().numpy(),
                                       inp.v_cache.float().numpy(), inp.page_table.numpy(),
                                       inp.context_lens.numpy(), cfg["hq"], cfg["hkv"], inp.scale,
                                       inp.page_size)
    for key, (o, lse) in outs.items():
        compare(o, ref, False, label=f"decode O {key} (all {ref.size} elements)")
        lg = lse.cpu().double().numpy()
        assert np.abs(lg - ref_lse).max() < 2e-3


def test_full_paged_decode_fp8():
    """The e4m3 cache of the benchmark (heads-outer layout, split + merge and
    monolithic) against the oracle on its dequantised values, every element."""
    import deterministic_flash_attention_amd as dfa
    cfg = synth.PAGED_DECODE
    inp = synth.decode_inputs(0, cfg["batch"], cfg["hq"], cfg["hkv"], cfg["d"],
                              ctx_min=cfg["ctx_min"], ctx_max=cfg["ctx_max"],
                              spare_pages=cfg["spare_pages"], dtype="fp8")
    mc = int(inp.context_lens.max())
    note(f"full fp8 decode: sum ctx = {int(inp.context_lens.sum())}")
    kc = dev(inp.k_cache.permute(0, 2, 1, 3))
    vc = dev(inp.v_cache.permute(0, 2, 1, 3))
    desc = (inp.q_scale, inp.k_scale, inp.v_scale)
    o_split = dfa.decode(dev(inp.q), kc, vc, dev(inp.page_table), dev(inp.context_lens), mc,
                         softmax_scale=inp.scale, schedule=SPLIT, descales=desc, kv_layout="HND")
    o_mono = dfa.decode(dev(inp.q), kc, vc, dev(inp.page_table), dev(inp.context_lens), mc,
                        softmax_scale=inp.scale, schedule=MONO, descales=desc, kv_layout="HND")
    torch.cuda.synchronize()
    assert_bitwise(o_split, o_mono, "fp8 decode split vs monolithic")
    note("oracle on every sequence")
    ref, _ = oracle.paged_decode(oracle.dequantize_e4m3(inp.q.numpy(), inp.q_scale),
                                 oracle.dequantize_e4m3(inp.k_cache.numpy(), inp.k_scale),
                                 oracle.dequantize_e4m3(inp.v_cache.numpy(), inp.v_scale),
                                 inp.page_table.numpy(), inp.context_lens.numpy(), cfg["hq"],
                                 cfg["hkv"], inp.scale, inp.page_size)
    compare(o_split, ref, True, label=f"fp8 decode O (all {ref.size} elements)")
