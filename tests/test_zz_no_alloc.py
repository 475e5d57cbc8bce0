"""The allocation-free paged decode (attn_decode_fwd_noalloc): split decode and
merge in one call with the partials in the library's static device scratch.
Its output must equal the existing entry points' (attn_decode_split_fwd split +
attn_chunk_merge with a caller workspace) bit for bit, on consecutive calls
whose second input is smaller (so a call never reads what an earlier call left
in the scratch), and match the oracle at the bf16 / fp8 tolerances."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_utils import assert_bitwise, compare, dev, note

pytestmark = pytest.mark.gpu

SPLIT = 1


def _run_both(inp, layout="NHD"):
    import deterministic_flash_attention_amd as dfa
    kc, vc = inp.k_cache, inp.v_cache
    if layout == "HND":
        kc, vc = kc.permute(0, 2, 1, 3), vc.permute(0, 2, 1, 3)
    q, kc, vc = dev(inp.q), dev(kc), dev(vc)
    pt, cl = dev(inp.page_table), dev(inp.context_lens)
    mc = int(inp.context_lens.max())
    desc = (inp.q_scale, inp.k_scale, inp.v_scale)
    ref, ref_lse = dfa.decode(q, kc, vc, pt, cl, mc, softmax_scale=inp.scale, schedule=SPLIT,
                              descales=desc, return_lse=True, kv_layout=layout)
    o = torch.full_like(ref, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    dfa.attn_decode_fwd_noalloc(q, kc, vc, pt, cl, mc, inp.scale, o, lse, descales=desc,
                                kv_layout=layout)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return o, lse, ref, ref_lse


def _oracle(inp):
    if inp.dtype == "fp8":
        q = oracle.dequantize_e4m3(inp.q.numpy(), inp.q_scale)
        kc = oracle.dequantize_e4m3(inp.k_cache.numpy(), inp.k_scale)
        vc = oracle.dequantize_e4m3(inp.v_cache.numpy(), inp.v_scale)
    else:
        q, kc, vc = synth.to_f64(inp.q), inp.k_cache.float().numpy(), inp.v_cache.float().numpy()
    return oracle.paged_decode(q, kc, vc, inp.page_table.numpy(), inp.context_lens.numpy(),
                               inp.hq, inp.hkv, inp.scale, inp.page_size)


def test_noalloc_decode_consecutive_calls():
    cfg = synth.PAGED_DECODE
    # 1: the full paged decode workload (64 sequences, contexts up to 32768).
    big = synth.decode_inputs(0, cfg["batch"], cfg["hq"], cfg["hkv"], cfg["d"],
                              ctx_min=cfg["ctx_min"], ctx_max=cfg["ctx_max"],
                              spare_pages=cfg["spare_pages"])
    note(f"noalloc call 1: full workload, sum ctx {int(big.context_lens.sum())}")
    o, lse, ref, ref_lse = _run_both(big, "HND")
    assert_bitwise(o, ref, "noalloc O vs split + merge (call 1)")
    assert_bitwise(lse, ref_lse, "noalloc lse vs split + merge (call 1)")
    # 2: a smaller batch right after it, with fewer chunks and an empty sequence.
    small = synth.decode_inputs(5, 5, 8, 2, 128, context_lens=[1, 100, 513, 2000, 0],
                                spare_pages=4)
    note("noalloc call 2: 5 sequences")
    o, lse, ref, ref_lse = _run_both(small)
    assert_bitwise(o, ref, "noalloc O vs split + merge (call 2)")
    assert_bitwise(lse, ref_lse, "noalloc lse vs split + merge (call 2)")
    want, _ = _oracle(small)
    compare(o, want, False, label="noalloc call 2 vs oracle")
    assert torch.all(o[4].float() == 0) and torch.all(torch.isneginf(lse[4]))
    # 3: e4m3 cache, smaller again.
    fp8 = synth.decode_inputs(6, 3, 4, 4, 192, context_lens=[700, 1, 1500], spare_pages=2,
                              dtype="fp8")
    note("noalloc call 3: e4m3, 3 sequences, D=192")
    o, lse, ref, ref_lse = _run_both(fp8)
    assert_bitwise(o, ref, "noalloc O vs split + merge (call 3, e4m3)")
    want, _ = _oracle(fp8)
    compare(o, want, True, label="noalloc call 3 vs oracle")


def test_noalloc_rejects_oversized_partials():
    """Partials beyond the static scratch: DA_EWORKSPACE, nothing written."""
    import deterministic_flash_attention_amd as dfa
    inp = synth.decode_inputs(7, 2, 32, 8, 128, context_lens=[10, 20], spare_pages=1)
    o = torch.full((2, 32, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    # 2 rows x 32 heads x 8192 chunks x 130 x 4 B > 128 MiB; the page table is
    # checked only against the claimed maximum context length on the host.
    mc = 8192 * 512
    pt = torch.zeros(2, mc // 16, dtype=torch.int32)
    pt[:, :inp.page_table.shape[1]] = inp.page_table
    assert dfa.attn_partials_bytes(2, 32, dfa.attn_num_chunks(mc), 128) > dfa.DECODE_SCRATCH_BYTES
    with pytest.raises(dfa.DetAttnError) as err:
        dfa.attn_decode_fwd_noalloc(dev(inp.q), dev(inp.k_cache), dev(inp.v_cache), dev(pt),
                                    dev(inp.context_lens), mc, inp.scale, o)
    assert err.value.status == 3  # DA_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.all(o.float() == 3.0)
