"""Bitwise invariance of the HIP path across schedules and batch composition
(RL-Kernel page, section 2: the monolithic and split schedules are
bit-identical, which is what makes decode agree with training; its test file
covers prefill-vs-decode identity, batch composition and the unmasked fast
path).  Also the store bounds: sentinel pre-fill outside the valid cells and
the padded-row alias set (FlyDSL conv3d page, "Root cause"; aiter MQA-logits
page, "Correctness")."""
import numpy as np
import pytest
import torch

import synth
from alias_sets import packed_alias_rows
from gpu_utils import assert_bitwise, dev, note, run_decode, run_prefill

pytestmark = pytest.mark.gpu

MONO, SPLIT = 0, 1


def _prefill(inp, schedule, **kw):
    return run_prefill(inp, schedule, **kw)


@pytest.mark.parametrize("case", [
    ([300], None, 2, 1, 64, True, "bf16"),
    ([600, 250, 1, 397], None, 8, 2, 128, True, "bf16"),
    ([1100], None, 4, 4, 128, False, "bf16"),
    ([100, 1, 37], [700, 513, 64], 4, 2, 128, True, "bf16"),
    ([700], None, 4, 4, 192, True, "fp8"),
    ([700], None, 4, 4, 192, False, "fp8"),
])
def test_split_equals_monolithic_prefill(case):
    sq, sk, hq, hkv, d, causal, dt = case
    inp = synth.prefill_inputs(31, sq, hq, hkv, d, causal, seqlens_k=sk, dtype=dt)
    note(f"split vs mono {case}")
    o1, l1 = _prefill(inp, MONO, return_lse=True)
    o2, l2 = _prefill(inp, SPLIT, return_lse=True)
    assert_bitwise(o1, o2, "O split vs monolithic")
    assert_bitwise(l1, l2, "lse split vs monolithic")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_split_equals_monolithic_decode(dtype):
    ctx = [1, 17, 64, 65, 512, 513, 1200, 3000]
    inp = synth.decode_inputs(33, len(ctx), 16, 4, 128, context_lens=ctx, spare_pages=8, dtype=dtype)
    o1, l1 = run_decode(inp, MONO, return_lse=True)
    o2, l2 = run_decode(inp, SPLIT, return_lse=True)
    assert_bitwise(o1, o2, "decode O split vs monolithic")
    assert_bitwise(l1, l2, "decode lse split vs monolithic")


@pytest.mark.parametrize("dtype,d,hq,hkv", [("bf16", 128, 8, 2), ("bf16", 64, 8, 2),
                                            ("bf16", 192, 8, 2), ("fp8", 192, 8, 2),
                                            ("fp8", 128, 8, 2), ("fp8", 64, 8, 2),
                                            ("bf16", 128, 32, 1), ("fp8", 128, 4, 4)])
def test_decode_equals_last_prefill_row(dtype, d, hq, hkv):
    """The decode token of a sequence of length L equals row L-1 of its causal
    prefill, bit for bit, for lengths around block and chunk boundaries (groups
    of 4, of 32 query heads per kv head, and of one)."""
    lens = [1, 2, 63, 64, 65, 511, 512, 513, 1000, 1537]
    inp = synth.prefill_inputs(35, lens, hq, hkv, d, True, dtype=dtype)
    o_pre = _prefill(inp, MONO)
    # Page the same K/V into a shuffled paged cache; the decode query is the last row.
    ps = 16
    pages = [(n + ps - 1) // ps for n in lens]
    npages = sum(pages) + 5
    perm = torch.randperm(npages, generator=torch.Generator().manual_seed(3))
    kc = torch.zeros(npages, ps, hkv, d, dtype=inp.k.dtype)
    vc = torch.zeros_like(kc)
    table = torch.zeros(len(lens), max(pages), dtype=torch.int32)
    cu = inp.cu_seqlens_k.tolist()
    pos = 0
    for b, n in enumerate(lens):
        for j in range(pages[b]):
            table[b, j] = int(perm[pos])
            pos += 1
        for t in range(n):
            kc[table[b, t // ps], t % ps] = inp.k[cu[b] + t]
            vc[table[b, t // ps], t % ps] = inp.v[cu[b] + t]
    last = torch.tensor([cu[b + 1] - 1 for b in range(len(lens))])
    qd = inp.q[last].contiguous()
    dec = synth.DecodeInputs(qd, kc, vc, table, torch.tensor(lens, dtype=torch.int32), hq, hkv, d,
                             ps, inp.scale, 0, dtype, inp.q_scale, inp.k_scale, inp.v_scale)
    for sched in (SPLIT, MONO):
        o_dec = run_decode(dec, sched)
        assert_bitwise(o_dec, o_pre[last.to(o_pre.device)], f"decode({sched}) vs last prefill row")


def test_batch_composition_and_order():
    """A sequence's rows do not depend on the other sequences in the batch."""
    lens = [600, 250, 1, 397, 130]
    hq, hkv, d = 8, 2, 128
    inp = synth.prefill_inputs(37, lens, hq, hkv, d, True)
    o_all = _prefill(inp, MONO).cpu()
    cu = inp.cu_seqlens_q.tolist()
    for b, n in enumerate(lens):
        sub = synth.PrefillInputs(inp.q[cu[b]:cu[b + 1]], inp.k[cu[b]:cu[b + 1]],
                                  inp.v[cu[b]:cu[b + 1]], synth.cu_seqlens([n]),
                                  synth.cu_seqlens([n]), [n], [n], hq, hkv, d, inp.scale, True)
        o_one = _prefill(sub, MONO).cpu()
        assert_bitwise(o_one, o_all[cu[b]:cu[b + 1]], f"sequence {b} alone vs in batch")
    # reversed batch order
    order = list(reversed(range(len(lens))))
    rq = torch.cat([inp.q[cu[b]:cu[b + 1]] for b in order])
    rk = torch.cat([inp.k[cu[b]:cu[b + 1]] for b in order])
    rv = torch.cat([inp.v[cu[b]:cu[b + 1]] for b in order])
    rl = [lens[b] for b in order]
    rev = synth.PrefillInputs(rq, rk, rv, synth.cu_seqlens(rl), synth.cu_seqlens(rl), rl, rl, hq,
                              hkv, d, inp.scale, True)
    o_rev = _prefill(rev, SPLIT).cpu()
    rcu = synth.cu_seqlens(rl).tolist()
    for i, b in enumerate(order):
        assert_bitwise(o_rev[rcu[i]:rcu[i + 1]], o_all[cu[b]:cu[b + 1]], f"seq {b} reordered")


def test_decode_batch_composition():
    ctx = [5, 900, 64, 2100]
    inp = synth.decode_inputs(39, len(ctx), 8, 2, 128, context_lens=ctx, spare_pages=4)
    o_all = run_decode(inp, SPLIT).cpu()
    for b in range(len(ctx)):
        one = synth.DecodeInputs(inp.q[b:b + 1], inp.k_cache, inp.v_cache, inp.page_table[b:b + 1],
                                 inp.context_lens[b:b + 1], 8, 2, 128, 16, inp.scale)
        assert_bitwise(run_decode(one, SPLIT).cpu(), o_all[b:b + 1], f"decode seq {b} alone")


def test_unmasked_fast_path_equals_masked_path():
    """The last row of a causal sequence sees every key, as does every row of
    the dense run; in the causal run the last tile's diagonal blocks take the
    masked path, in the dense run all blocks take the fast path."""
    for n in (1024, 1000, 777):
        inp_c = synth.prefill_inputs(41, [n], 4, 2, 128, True)
        inp_d = synth.prefill_inputs(41, [n], 4, 2, 128, False)
        oc = _prefill(inp_c, MONO)
        od = _prefill(inp_d, MONO)
        assert_bitwise(oc[n - 1], od[n - 1], f"last row causal vs dense n={n}")


def test_repeat_runs_bitwise():
    inp = synth.prefill_inputs(43, [600, 250, 1, 397], 8, 2, 128, True)
    ref = _prefill(inp, MONO)
    for _ in range(4):
        assert_bitwise(_prefill(inp, MONO), ref, "repeat monolithic")
        assert_bitwise(_prefill(inp, SPLIT), ref, "repeat split")


def test_closed_form_rows_bitwise():
    """Causal row 0 and a length-1 sequence see one key: O = V[that key] exactly."""
    lens = [300, 1, 129]
    inp = synth.prefill_inputs(45, lens, 4, 2, 64, True)
    o = _prefill(inp, MONO).cpu()
    cu = inp.cu_seqlens_q.tolist()
    for b in range(3):
        for h in range(4):
            assert_bitwise(o[cu[b], h], inp.v[cu[b], h // 2], f"row 0 of seq {b} head {h}")
    dec = synth.decode_inputs(47, 3, 4, 1, 128, context_lens=[1, 1, 1], spare_pages=2)
    od = run_decode(dec, SPLIT).cpu()
    for b in range(3):
        page = int(dec.page_table[b, 0])
        for h in range(4):
            assert_bitwise(od[b, h], dec.v_cache[page, 0, 0], f"decode ctx=1 seq {b}")


def test_sentinel_survives_outside_valid_rows():
    """O pre-filled with NaN plus guard rows before and after; only the rows of
    the sequences are written, the guards and an unowned tail keep the NaN."""
    lens = [300, 1, 129]
    hq, hkv, d = 4, 2, 64
    inp = synth.prefill_inputs(49, lens, hq, hkv, d, True)
    total = sum(lens)
    guard = 200
    for sched in (MONO, SPLIT):
        extra = 50 if sched == MONO else 0  # unowned rows only for the monolithic schedule
        buf = torch.full((total + 2 * guard + extra, hq, d), float("nan"), dtype=torch.bfloat16,
                         device="cuda")
        q = torch.cat([inp.q, torch.zeros(extra, hq, d, dtype=inp.q.dtype)])
        pinp = synth.PrefillInputs(q, inp.k, inp.v, inp.cu_seqlens_q, inp.cu_seqlens_k, lens, lens,
                                   hq, hkv, d, inp.scale, True)
        out = buf[guard:guard + total + extra]
        run_prefill(pinp, sched, out=out)
        assert not torch.isnan(out[:total].float()).any()
        assert torch.isnan(out[total:].float()).all(), "unowned rows were written"
        assert torch.isnan(buf[:guard].float()).all(), "guard before O was written"
        assert torch.isnan(buf[guard + total + extra:].float()).all(), "guard after O was written"


def test_padded_rows_do_not_alias_next_sequence():
    """Each sequence is run alone (batch of one, via an offset cu_seqlens view)
    into the shared packed O after its successors were written; the rows that
    an unguarded store of its tail tile would hit (predicted set) must keep the
    successors' values."""
    lens = [4096, 2500, 1, 3969]
    hq, hkv, d = 2, 1, 128
    import deterministic_flash_attention_amd as dfa
    inp = synth.prefill_inputs(51, lens, hq, hkv, d, True)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    cq, ck = dev(inp.cu_seqlens_q), dev(inp.cu_seqlens_k)
    ref = dfa.prefill(q, k, v, cq, ck, max(lens), max(lens), True)
    out = torch.full_like(ref, float("nan"))
    for b in reversed(range(len(lens))):
        dfa.attn_prefill_fwd(q, k, v, cq[b:b + 2], ck[b:b + 2], lens[b], lens[b],
                             1.0 / np.sqrt(d), True, dfa.MONOLITHIC, o=out)
    torch.cuda.synchronize()
    assert_bitwise(out, ref, "sequences written one by one, last to first")
    alias = packed_alias_rows(lens, 128)
    assert sum(len(r) for r, _ in alias) == 60 + 127  # the predicted clobber set is non-empty


@pytest.mark.parametrize("d", [64, 192])
def test_e4m3_widening_every_code(d):
    """A query that sees a single key returns that key's V row exactly (p = 1,
    l = 1).  V rows holding all 256 E4M3FN codes pin the exact e4m3 -> bf16
    widening of the V stage against the OCP decoding the oracle writes out
    (NaN codes give NaN), through prefill and through the paged decode."""
    import oracle
    nrows = 256 // d + (1 if 256 % d else 0)
    lens = [1] * nrows
    inp = synth.prefill_inputs(61, lens, 1, 1, d, True, dtype="fp8")
    codes = torch.arange(nrows * d, dtype=torch.int64) % 256
    v = codes.to(torch.uint8).reshape(nrows, 1, d)
    inp = synth.PrefillInputs(inp.q, inp.k, v, inp.cu_seqlens_q, inp.cu_seqlens_k, lens, lens, 1, 1,
                              d, inp.scale, True, "fp8", inp.q_scale, inp.k_scale, 1.0, inp.seed)
    # The accumulator starts at +0 and +0 + (-0) = +0, so the -0 code comes out as +0.
    table = oracle.e4m3fn_table()[codes.numpy()] + 0.0
    want = torch.from_numpy(table).to(torch.bfloat16).reshape(nrows, 1, d)
    nan = torch.isnan(want)
    assert nan.any() and not nan.all()
    for sched in (MONO, SPLIT):
        note(f"e4m3 widening d={d} schedule={sched}")
        o = _prefill(inp, sched).cpu()
        assert torch.isnan(o[nan]).all(), "NaN codes must widen to NaN"
        assert_bitwise(o[~nan], want[~nan], f"prefill schedule {sched}")
    kc = inp.k.reshape(nrows, 1, 1, d).expand(nrows, 16, 1, d).contiguous()
    vc = v.reshape(nrows, 1, 1, d).expand(nrows, 16, 1, d).contiguous()
    pages = torch.arange(nrows, dtype=torch.int32).reshape(nrows, 1)
    dec = synth.DecodeInputs(inp.q.contiguous(), kc, vc, pages, torch.ones(nrows, dtype=torch.int32),
                             1, 1, d, 16, inp.scale, 0, "fp8", inp.q_scale, inp.k_scale, 1.0)
    for sched in (SPLIT, MONO):
        o = run_decode(dec, sched).cpu().reshape(nrows, 1, d)
        assert torch.isnan(o[nan]).all(), "NaN codes must widen to NaN"
        assert_bitwise(o[~nan], want[~nan], f"decode schedule {sched}")


def _zero_sign_inputs():
    """One sequence of 200 keys (D=64, one head) built so that row 100's
    accumulator holds -0 in column 5 before a block that is fully masked for
    it: its block-0 scores are O(10) (log2 units) and V[:, 5] = -1 there, so
    acc[5] < 0; key 90 scores about 288 (log2 units), so at block 1 alpha =
    exp2(m - m') underflows to 0, acc[5] * 0 = -0, and every product of block 1
    in that column is -0 (p = 1 times V[90, 5] = -0, p = 0 times -1).  Keys from
    128 on have V[:, 5] = +1, so a computed fully masked block 2 adds +0 products
    and can turn that -0 into +0."""
    n, d, r, ks, col = 200, 64, 100, 90, 5
    inp = synth.prefill_inputs(71, [n], 1, 1, d, True)
    q, k, v = inp.q.clone(), inp.k.clone(), inp.v.clone()
    q[r, 0] = 0.0
    q[r, 0, 0] = 40.0
    k[ks, 0] = 0.0
    k[ks, 0, 0] = 40.0
    v[:128, 0, col] = -1.0
    v[ks, 0, col] = -0.0
    v[128:, 0, col] = 1.0
    return q, k, v, n, d, r, ks, col, inp.scale


def test_zero_sign_under_alpha_underflow():
    """Fully masked blocks leave a row untouched (RL-Kernel page, section 2)
    up to the sign of zero, which the finalize step canonicalises: the prefill
    tiling (row 100's wave stops at block 1), the extend tiling with one cached
    token less of queries (row 100's wave reaches block 2, fully masked for
    it), split or monolithic, the paged extend and the decode of the same row
    agree bit for bit, and the row equals V[90] with the -0 written as +0."""
    import deterministic_flash_attention_amd as dfa
    q, k, v, n, d, r, ks, col, scale = _zero_sign_inputs()
    pre = synth.PrefillInputs(q, k, v, synth.cu_seqlens([n]), synth.cu_seqlens([n]), [n], [n],
                              1, 1, d, scale, True)
    o_pre = run_prefill(pre, MONO).cpu()
    ext = synth.PrefillInputs(q[1:].contiguous(), k, v, synth.cu_seqlens([n - 1]),
                              synth.cu_seqlens([n]), [n - 1], [n], 1, 1, d, scale, True)
    want = v[ks, 0].clone()
    want[col] = 0.0  # +0: the canonical zero
    assert_bitwise(o_pre[r, 0], want, "prefill row 100 = V[90] with +0")
    for sched in (MONO, SPLIT):
        o_ext = run_prefill(ext, sched).cpu()
        assert_bitwise(o_ext[r - 1], o_pre[r], f"extend (schedule {sched}) vs prefill row")
        assert_bitwise(o_ext, o_pre[1:], f"every extend row (schedule {sched}) vs prefill")
    # The same row as a decode step over a paged copy of keys 0..100, and
    # as a row of a paged extend launch.
    ps = 16
    npg = (n + ps - 1) // ps
    kc = torch.zeros(npg, ps, 1, d, dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    kc.view(-1, 1, d)[:n] = k
    vc.view(-1, 1, d)[:n] = v
    table = torch.arange(npg, dtype=torch.int32).reshape(1, npg)
    dec = synth.DecodeInputs(q[r:r + 1].contiguous(), kc, vc, table,
                             torch.tensor([r + 1], dtype=torch.int32), 1, 1, d, ps, scale)
    for sched in (SPLIT, MONO):
        assert_bitwise(run_decode(dec, sched).cpu()[0], o_pre[r], f"decode (schedule {sched})")
    pext = synth.ExtendInputs(q[1:].contiguous(), synth.cu_seqlens([n - 1]), None, k, v,
                              synth.cu_seqlens([n]), kc, vc, table,
                              torch.tensor([n], dtype=torch.int32), [n - 1], [n], 1, 1, d, ps,
                              scale, True)
    from gpu_utils import run_extend
    for sched in (MONO, SPLIT):
        assert_bitwise(run_extend(pext, sched).cpu(), o_pre[1:], f"paged extend (schedule {sched})")


def _threshold_inputs():
    """One head, D = 64, 1024 keys (two chunks), no mask.  Query row 300 holds
    8 in dimension 0 and zeros elsewhere; in dimension 0 every key is zero
    except one key per block, so in log2 units (scale 1/8, c = log2(e)/8) row
    300's block maxima are 1.4427 * 8 * y for the chosen y.  Within chunk 0 the
    reference starts at 0 and the maxima pass it by 7.93 (no move: P reaches
    2^7.93), 8.02 (a move), 7.93 and 8.02 again, then by 0 and 6.94 (no moves)
    before falling; chunk 1 starts from the empty state and repeats a no-move /
    move pair.  Every y is exact in bf16 and every decision has a margin of at
    least 0.025 over the fp32 roundings."""
    n, d, r = 1024, 64, 300
    inp = synth.prefill_inputs(83, [n], 1, 1, d, False)
    q, k = inp.q.clone(), inp.k.clone()
    q[r, 0] = 0.0
    q[r, 0, 0] = 8.0
    k[:, 0, 0] = 0.0
    ys = [0.0, 5.5, 5.5625, 11.0625, 11.125, 11.125, 15.9375, 2.0,
          2.0, 7.5, 7.5625, 0.0, 0.0, 0.0, 0.0, 0.0]
    for b, y in enumerate(ys):
        k[64 * b + 17, 0, 0] = y
    return synth.PrefillInputs(q, k, inp.v, synth.cu_seqlens([n]), synth.cu_seqlens([n]), [n], [n],
                               1, 1, d, inp.scale, False), r


def test_reference_threshold_edges():
    """The softmax reference moves only when a block's max passes it by more
    than 8 (log2 units); just below, P reaches 2^7.93 and the accumulator is
    not rescaled.  Against the oracle (the bound of the bf16 arithmetic,
    2^-8 (max|v| + |O|), as for the peaky rows), split = monolithic, and the
    decode of row 300 over a paged copy of the keys equals its prefill row."""
    import oracle
    from gpu_utils import oracle_inputs_prefill
    inp, r = _threshold_inputs()
    n, d = inp.q.shape[0], inp.q.shape[2]
    o_mono, lse = run_prefill(inp, MONO, return_lse=True)
    o_split = run_prefill(inp, SPLIT)
    assert_bitwise(o_split.cpu(), o_mono.cpu(), "split vs monolithic")
    q, k, v = oracle_inputs_prefill(inp)
    ref, ref_lse = oracle.attention(q, k, v, inp.cu_seqlens_q.numpy(), inp.cu_seqlens_k.numpy(),
                                    1, 1, inp.scale, False)
    g = o_mono.float().cpu().double().numpy()
    bound = 1.05 * 2.0**-8 * (float(np.abs(v).max()) + np.abs(ref)) + 1e-6
    err = np.abs(g - ref)
    note(f"threshold edges: row {r} max_abs={err[r].max():.3e}, all rows max err/bound="
         f"{float((err / bound).max()):.3f}")
    assert np.isfinite(g).all() and (err <= bound).all(), "beyond the bf16 arithmetic's bound"
    lse_err = np.abs(lse.cpu().double().numpy() - ref_lse)
    assert float(lse_err.max()) <= 2e-3, f"lse error {lse_err.max()}"
    ps = 16
    kc = inp.k.reshape(n // ps, ps, 1, d).contiguous()
    vc = inp.v.reshape(n // ps, ps, 1, d).contiguous()
    table = torch.arange(n // ps, dtype=torch.int32).reshape(1, n // ps)
    dec = synth.DecodeInputs(inp.q[r:r + 1].contiguous(), kc, vc, table,
                             torch.tensor([n], dtype=torch.int32), 1, 1, d, ps, inp.scale)
    for sched in (SPLIT, MONO):
        assert_bitwise(run_decode(dec, sched).cpu()[0], o_mono.cpu()[r], f"decode (schedule {sched})")
