"""Evidence for keeping P V on bf16 operands in the e4m3 kernels by default.

The option "P in e4m3 with l summed from the quantised P" may ship only if it
stays within the fp8 bar (max_abs <= 6e-2 against the oracle on the
dequantised inputs) across seeds.  This CPU test emulates the kernels'
arithmetic order in fp32 (scores, 64-key blocks inside 512-key chunks from the
empty state, online softmax with exp2, the ascending chunk fold, one bf16
rounding of O) on the first 1024 causal rows of 8 heads of the fp8 D=192
workload, for P rounded to bf16 (what the kernels do) and for P * 2^8 rounded to
E4M3FN (the rejected option; the 2^8 keeps small probabilities normal), and
compares both with the fp64 oracle.  It is an emulation, not the GPU kernel:
its sums run in PyTorch's order.  Causal early rows weigh two or three keys,
where P's 3-bit mantissa alone moves O by a few percent of the difference of
two V rows; in this emulation that lands at 0.043-0.056 over seeds 0-3 (8
heads), 0.033-0.056 over seeds 4-15, under the bar by a margin of 7% or less,
against 0.008-0.011 with P in bf16.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

ROWS, HEADS, SEEDS = 1024, 8, (0, 1, 2, 3)
BAR = 6e-2


def _e4m3_p(p):
    """P * 2^8 rounded to nearest even into E4M3FN, back to fp32 / 2^8."""
    return (p * 256.0).to(torch.float8_e4m3fn).to(torch.float32) / 256.0


def _emulate(qv, kv, vv, c, vscale, fp8_p):
    """qv [H, R, D], kv/vv [H, K, D] fp32 code values; causal with L_q = L_k."""
    h, r, d = qv.shape
    s_all = torch.bmm(qv, kv.transpose(1, 2).contiguous())  # raw dot products, fp32
    rows = torch.arange(r)[:, None]
    M = torch.full((h, r), -math.inf)
    L = torch.zeros(h, r)
    A = torch.zeros(h, r, d)
    for c0 in range(0, r, 512):
        m = torch.full((h, r), -math.inf)
        l = torch.zeros(h, r)
        acc = torch.zeros(h, r, d)
        for b0 in range(c0, min(c0 + 512, r), 64):
            keys = torch.arange(b0, b0 + 64)[None, :]
            s = torch.where(keys <= rows, s_all[:, :, b0:b0 + 64], torch.tensor(-math.inf))
            mb = s.max(dim=2).values * c
            mn = torch.maximum(m, mb)
            empty = mn == -math.inf
            alpha = torch.where(empty, torch.ones_like(mn), torch.exp2(m - mn))
            nms = torch.where(empty, torch.zeros_like(mn), -mn)
            p = torch.exp2(torch.addcmul(nms[..., None], s, torch.full_like(s, c)))
            pq = _e4m3_p(p) if fp8_p else p.to(torch.bfloat16).to(torch.float32)
            l = l * alpha + (pq if fp8_p else p).sum(dim=2)
            acc = acc * alpha[..., None] + torch.bmm(pq, vv[:, b0:b0 + 64, :])
            m = mn
        live = m > -math.inf
        Mn = torch.maximum(M, m)
        ca = torch.where(M == -math.inf, torch.zeros_like(M), torch.exp2(M - Mn))
        cb = torch.exp2(m - Mn)
        L = torch.where(live, L * ca + l * cb, L)
        A = torch.where(live[..., None], A * ca[..., None] + acc * cb[..., None], A)
        M = torch.where(live, Mn, M)
    o = torch.where(L[..., None] > 0, A / L[..., None], torch.zeros_like(A)) * vscale
    return o.to(torch.bfloat16).double().numpy()


def _errors(seed):
    cfg = synth.FP8_WIDE
    inp = synth.prefill_inputs(seed, cfg["seqlens"], cfg["hq"], cfg["hkv"], cfg["d"], True,
                               dtype="fp8")
    tab = torch.from_numpy(oracle.e4m3fn_table()).float()
    codes = lambda t: tab[t[:ROWS, :HEADS].long()].permute(1, 0, 2).contiguous()  # noqa: E731
    qv, kv, vv = codes(inp.q), codes(inp.k), codes(inp.v)
    c = float(np.float32(inp.scale * inp.q_scale * inp.k_scale * math.log2(math.e)))
    q = oracle.dequantize_e4m3(inp.q[:ROWS, :HEADS].numpy(), inp.q_scale)
    k = oracle.dequantize_e4m3(inp.k[:ROWS, :HEADS].numpy(), inp.k_scale)
    v = oracle.dequantize_e4m3(inp.v[:ROWS, :HEADS].numpy(), inp.v_scale)
    ref, _ = oracle.attention(q, k, v, [0, ROWS], [0, ROWS], HEADS, HEADS, inp.scale, True)
    ref = ref.transpose(1, 0, 2)
    out = {}
    for name, fp8_p in (("bf16_p", False), ("e4m3_p", True)):
        o = _emulate(qv, kv, vv, c, inp.v_scale, fp8_p)
        out[name] = float(np.abs(o - ref).max())
    return out


@pytest.fixture(scope="module")
def errors():
    return {s: _errors(s) for s in SEEDS}


def test_bf16_p_within_fp8_bar_with_margin(errors):
    for s, e in errors.items():
        print(f"seed {s}: P in bf16 max_abs {e['bf16_p']:.4f}, P in e4m3 {e['e4m3_p']:.4f}")
        assert e["bf16_p"] < BAR / 3, (s, e)


def test_e4m3_p_margin_is_thin(errors):
    """The option: P in e4m3 with l from the quantised P stays under 6e-2 in
    this emulation, but within 15% of the bar in some seed, and costs at least
    four times the error of bf16 P in every seed."""
    worst = max(e["e4m3_p"] for e in errors.values())
    assert 0.85 * BAR < worst < BAR, worst
    for s, e in errors.items():
        assert e["e4m3_p"] > 4 * e["bf16_p"], (s, e)
