"""Seeded input generators: determinism, shapes, page tables, fp8 codes."""
import numpy as np
import torch

import oracle
import synth


def test_prefill_inputs_deterministic():
    a = synth.prefill_inputs(3, [300], 2, 1, 64, True)
    b = synth.prefill_inputs(3, [300], 2, 1, 64, True)
    c = synth.prefill_inputs(4, [300], 2, 1, 64, True)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert not torch.equal(a.q, c.q)
    assert a.q.shape == (300, 2, 64) and a.k.shape == (300, 1, 64) and a.q.dtype == torch.bfloat16
    assert a.cu_seqlens_q.tolist() == [0, 300] and abs(a.scale - 0.125) < 1e-12


def test_varlen_cu_seqlens():
    x = synth.prefill_inputs(0, [4096, 2500, 1, 3969], 4, 1, 16, True)
    assert x.cu_seqlens_q.tolist() == [0, 4096, 6596, 6597, 10566]
    assert x.q.shape[0] == 10566


def test_unscaled_normal_values():
    x = synth.prefill_inputs(0, [4096], 4, 4, 64, False)
    q = x.q.float()
    assert abs(q.mean().item()) < 0.01 and abs(q.std().item() - 1.0) < 0.01


def test_fp8_codes_round_to_nearest():
    x = synth.prefill_inputs(1, [257], 2, 2, 192, False, dtype="fp8")
    assert x.q.dtype == torch.uint8 and x.dtype == "fp8"
    # regenerate the fp32 source and check each code is a nearest E4M3FN value of x/scale
    g = torch.Generator().manual_seed(1)
    src = torch.randn(257, 2, 192, generator=g).double().numpy()
    t = oracle.e4m3fn_table()
    deq = t[x.q.numpy()]
    y = src / np.float32(x.q_scale)
    finite = np.sort(np.unique(t[np.isfinite(t)]))
    idx = np.clip(np.searchsorted(finite, y), 1, len(finite) - 1)
    best = np.minimum(np.abs(finite[idx] - y), np.abs(finite[idx - 1] - y))
    assert np.all(np.abs(deq - y) <= best + 1e-12)
    assert np.abs(deq).max() == 448.0


def test_decode_page_table_and_poison():
    x = synth.decode_inputs(5, 6, 8, 2, 16, context_lens=[1, 16, 17, 100, 33, 2], spare_pages=5)
    pages = [1, 1, 2, 7, 3, 1]
    used = np.concatenate([x.page_table[b, :n].numpy() for b, n in enumerate(pages)])
    assert len(np.unique(used)) == len(used) == sum(pages)
    assert x.k_cache.shape == (sum(pages) + 5, 16, 2, 16)
    for b, ctx in enumerate([1, 16, 17, 100, 33, 2]):
        kb = oracle.gather_pages(x.k_cache.float().numpy(), x.page_table[b].numpy(), ctx, 16)
        assert np.isfinite(kb).all()
    # a dead slot right after the context is NaN
    p = int(x.page_table[0, 0])
    assert torch.isnan(x.k_cache[p, 1].float()).all() and torch.isnan(x.v_cache[p, 1].float()).all()
    # table entries past a sequence's pages point at spare (poisoned) pages
    spare = set(range(x.k_cache.shape[0])) - set(used.tolist())
    assert int(x.page_table[0, 3]) in spare
