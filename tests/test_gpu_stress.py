"""Bitwise repeat stress of the full-size prefill workloads: 200 launches each,
every output pre-filled with NaN and compared bit for bit with the first run,
stopping at the first mismatch (FlyDSL conv3d page, "Verification": an
intermittent store race showed only over many repetitions).  The ping-pong
prefill depends on its LDS slot discipline between the two halves of the
workgroup, and the paged extend's spread tiles on exact vector-memory wait
counts for loads kept in flight across LDS-only barriers; a race there would
show here as a run-to-run difference."""
import pytest
import torch

import synth
from gpu_utils import bits, dev, note

pytestmark = pytest.mark.gpu

ITERS = 200


@pytest.mark.parametrize("cfg,causal", [(synth.DENSE_PREFILL, False),
                                        (synth.CAUSAL_VARLEN, True)])
def test_repeat_200_bitwise(cfg, causal):
    import deterministic_flash_attention_amd as dfa
    inp = synth.prefill_inputs(0, cfg["seqlens"], cfg["hq"], cfg["hkv"], cfg["d"], causal)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    cq, ck = dev(inp.cu_seqlens_q), dev(inp.cu_seqlens_k)
    ms, mk = max(inp.seqlens_q), max(inp.seqlens_k)
    ref = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    dfa.attn_prefill_fwd(q, k, v, cq, ck, ms, mk, inp.scale, causal, dfa.MONOLITHIC, o=ref)
    torch.cuda.synchronize()
    assert not torch.isnan(ref).any()
    ref_bits = bits(ref)
    out = torch.empty_like(ref)
    note(f"{cfg['name']}: {ITERS} repeats")
    for it in range(ITERS):
        out.fill_(float("nan"))
        dfa.attn_prefill_fwd(q, k, v, cq, ck, ms, mk, inp.scale, causal, dfa.MONOLITHIC, o=out)
        same = torch.equal(bits(out), ref_bits)
        if not same:
            diff = (bits(out) != ref_bits).nonzero()
            note(f"iteration {it}: {diff.shape[0]} elements differ, first at {diff[0].tolist()}")
        assert same, f"{cfg['name']}: run {it} differs from the first run"
    note(f"{cfg['name']}: {ITERS} repeats bitwise identical")


def test_mixed_paged_batch_spread_repeat_200_bitwise():
    """The mixed prefill / extend / decode batch over a paged cache with the
    chunk-spread workspace (its decode rows' chunks on spread tiles), 200
    launches, O and lse bit for bit, the counters back at zero every time."""
    import deterministic_flash_attention_amd as dfa
    cfg = synth.MIXED_EXTEND
    inp = synth.extend_inputs(0, cfg["ctx_lens"], cfg["q_lens"], cfg["hq"], cfg["hkv"], cfg["d"],
                              spare_pages=cfg["spare_pages"])
    q, cq = dev(inp.q), dev(inp.cu_seqlens_q)
    kc, vc, pt, cl = dev(inp.k_cache), dev(inp.v_cache), dev(inp.page_table), dev(inp.context_lens)
    mq, mc = max(inp.q_lens), max(inp.ctx_lens)
    nb = dfa.attn_extend_workspace_bytes(len(inp.q_lens), cfg["hq"], cfg["hkv"],
                                         dfa.attn_num_chunks(mc), cfg["d"])
    ws = torch.zeros((nb + 3) // 4, dtype=torch.float32, device="cuda")
    counters = ws[:65536].view(torch.int32)

    def run(o, lse):
        dfa.attn_paged_extend_fwd(q, cq, kc, vc, pt, cl, mq, mc, inp.scale, True, dfa.MONOLITHIC,
                                  o=o, lse=lse, partials=ws)

    ref = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    ref_lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    run(ref, ref_lse)
    torch.cuda.synchronize()
    assert not torch.isnan(ref).any()
    ref_bits, lse_bits = bits(ref), bits(ref_lse)
    out, out_lse = torch.empty_like(ref), torch.empty_like(ref_lse)
    note(f"mixed paged batch with the spread workspace: {ITERS} repeats")
    for it in range(ITERS):
        out.fill_(float("nan"))
        out_lse.fill_(float("nan"))
        run(out, out_lse)
        same = torch.equal(bits(out), ref_bits) and torch.equal(bits(out_lse), lse_bits)
        if not same:
            diff = (bits(out) != ref_bits).nonzero()
            note(f"iteration {it}: {diff.shape[0]} O elements differ")
        assert same, f"mixed paged batch: run {it} differs from the first run"
        assert int(torch.count_nonzero(counters)) == 0, f"run {it}: counters not back at zero"
    note(f"mixed paged batch: {ITERS} repeats bitwise identical")
