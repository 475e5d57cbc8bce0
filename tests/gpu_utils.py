"""Helpers for the GPU tests: move seeded inputs to the device, run the HIP path
through the C ABI, evaluate the oracle on the same stored values, compare."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import oracle.gemm as ogemm
import synth

BF16_MAX_ABS, BF16_MEAN_ABS = 1e-2, 1e-3  # tolerances for bf16 inputs
FP8_MAX_ABS = 6e-2                         # fp8 inputs, against the dequantised oracle


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().to("cuda")


def oracle_inputs_prefill(inp: synth.PrefillInputs):
    if inp.dtype == "fp8":
        q = oracle.dequantize_e4m3(inp.q.numpy(), inp.q_scale)
        k = oracle.dequantize_e4m3(inp.k.numpy(), inp.k_scale)
        v = oracle.dequantize_e4m3(inp.v.numpy(), inp.v_scale)
    else:
        q, k, v = synth.to_f64(inp.q), synth.to_f64(inp.k), synth.to_f64(inp.v)
    return q, k, v


def descales(inp) -> tuple:
    return (inp.q_scale, inp.k_scale, inp.v_scale)


def run_prefill(inp: synth.PrefillInputs, schedule: int, return_lse: bool = False, out=None):
    import deterministic_flash_attention_amd as dfa
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    cq, ck = dev(inp.cu_seqlens_q), dev(inp.cu_seqlens_k)
    res = dfa.prefill(q, k, v, cq, ck, max(inp.seqlens_q), max(inp.seqlens_k), inp.causal,
                      softmax_scale=inp.scale, schedule=schedule, descales=descales(inp),
                      out=out, return_lse=return_lse)
    torch.cuda.synchronize()
    return res


def run_decode(inp: synth.DecodeInputs, schedule: int, return_lse: bool = False, max_ctx=None):
    import deterministic_flash_attention_amd as dfa
    mc = int(inp.context_lens.max()) if max_ctx is None else max_ctx
    res = dfa.decode(dev(inp.q), dev(inp.k_cache), dev(inp.v_cache), dev(inp.page_table),
                     dev(inp.context_lens), mc, softmax_scale=inp.scale, schedule=schedule,
                     descales=descales(inp), return_lse=return_lse)
    torch.cuda.synchronize()
    return res


def extend_workspace(inp: synth.ExtendInputs):
    """A zero-filled workspace for the monolithic paged extend's chunk spread."""
    import deterministic_flash_attention_amd as dfa
    nbytes = dfa.attn_extend_workspace_bytes(len(inp.q_lens), inp.hq, inp.hkv,
                                             dfa.attn_num_chunks(max(inp.ctx_lens)), inp.d)
    return torch.zeros((nbytes + 3) // 4, dtype=torch.float32, device="cuda")


def run_extend(inp: synth.ExtendInputs, schedule: int, return_lse: bool = False, out=None,
               workspace=None, window=(-1, -1)):
    """The mixed batch through attn_paged_extend_fwd (plus the merge for SPLIT)."""
    import deterministic_flash_attention_amd as dfa
    res = dfa.paged_extend(dev(inp.q), dev(inp.cu_seqlens_q), dev(inp.k_cache), dev(inp.v_cache),
                           dev(inp.page_table), dev(inp.context_lens), max(inp.q_lens),
                           max(inp.ctx_lens), inp.causal, softmax_scale=inp.scale,
                           schedule=schedule, descales=descales(inp), out=out,
                           return_lse=return_lse, workspace=workspace, window=window)
    torch.cuda.synchronize()
    return res


def oracle_extend(inp: synth.ExtendInputs, rows=None, window=(-1, -1)):
    """fp64 oracle of a paged extend batch: each sequence's keys gathered from
    its pages by the oracle (over the sequence's own pages, widened to fp64),
    then the packed-varlen definition with bottom-right alignment (and the
    sliding window, if given)."""
    ps = inp.page_size

    ks, vs = [], []
    for b, c in enumerate(inp.ctx_lens):
        pages = inp.page_table[b, :(c + ps - 1) // ps].long()
        local = np.arange(len(pages))
        kp, vp = inp.k_cache[pages], inp.v_cache[pages]
        if inp.dtype == "fp8":
            kp = oracle.dequantize_e4m3(kp.numpy(), inp.k_scale)
            vp = oracle.dequantize_e4m3(vp.numpy(), inp.v_scale)
        else:
            kp, vp = synth.to_f64(kp), synth.to_f64(vp)
        ks.append(oracle.gather_pages(kp, local, c, ps))
        vs.append(oracle.gather_pages(vp, local, c, ps))
    if inp.dtype == "fp8":
        q = oracle.dequantize_e4m3(inp.q.numpy(), inp.q_scale)
    else:
        q = synth.to_f64(inp.q)
    return oracle.attention(q, np.concatenate(ks), np.concatenate(vs), inp.cu_seqlens_q.numpy(),
                            inp.cu_full.numpy(), inp.hq, inp.hkv, inp.scale, inp.causal,
                            rows=rows, window=window)


def compare(gpu_o: torch.Tensor, ref: np.ndarray, fp8: bool, rows=None, label: str = ""):
    """Element-wise comparison against the oracle at the stated tolerance.

    Returns (max_abs, mean_abs).  On failure reports the worst element, its
    reference value and the bf16 spacing there."""
    g = gpu_o.float().cpu().double().numpy()
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert np.isfinite(g).all(), f"{label}: non-finite GPU output"
    err = np.abs(g - ref)
    mx, mean = float(err.max()), float(err.mean())
    idx = np.unravel_index(int(err.argmax()), err.shape)
    ref_v = float(ref[idx])
    ulp = 2.0 ** (math.floor(math.log2(abs(ref_v))) - 7) if ref_v != 0 else 0.0
    note(f"{label}: max_abs={mx:.3e} mean_abs={mean:.3e} worst at {idx} ref={ref_v:.5f} "
         f"gpu={g[idx]:.5f} bf16_ulp={ulp:.2e}")
    if fp8:
        assert mx <= FP8_MAX_ABS, f"{label}: fp8 max_abs {mx} > {FP8_MAX_ABS}"
    else:
        assert mx <= BF16_MAX_ABS, f"{label}: max_abs {mx} > {BF16_MAX_ABS}"
        assert mean <= BF16_MEAN_ABS, f"{label}: mean_abs {mean} > {BF16_MEAN_ABS}"
    return mx, mean


def bits(t: torch.Tensor) -> torch.Tensor:
    """Raw bit pattern of a bf16/fp32 tensor (for bitwise comparisons)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def assert_bitwise(a: torch.Tensor, b: torch.Tensor, label: str) -> None:
    ba, bb = bits(a), bits(b)
    same = torch.equal(ba, bb)
    if not same:
        diff = (ba != bb).nonzero()
        note(f"{label}: {diff.shape[0]} differing elements, first at {diff[0].tolist()}")
    assert same, f"{label}: not bitwise identical"


# ---------------------------------------------------------------- GEMM
def gemm_views(inp: synth.GemmInputs, device="cuda"):
    """Device views of the (possibly row-padded) operands: A [M, K] with lda =
    the stored width, W [N, K] or [K, N] likewise."""
    a = inp.a.to(device)[:, :inp.k]
    w = inp.w.to(device)
    w = w[:, :inp.n] if inp.weight_kn else w[:, :inp.k]
    return a, w


def run_gemm(inp: synth.GemmInputs, schedule: int, config: int = -1, out=None, a=None):
    import deterministic_flash_attention_amd as dfa
    da, dw = gemm_views(inp)
    if a is not None:
        da = a
    c = dfa.gemm(da, dw, dfa.WEIGHT_KN if inp.weight_kn else dfa.WEIGHT_NK, schedule=schedule,
                 config=config, out=out)
    torch.cuda.synchronize()
    return c


def oracle_gemm(inp: synth.GemmInputs, rows=None):
    """fp64 product of the stored bf16 operands, and sum_k |a_ik| |b_kj| (the
    scale of the accumulation error bound)."""
    a = synth.to_f64(inp.a[:, :inp.k])
    w = synth.to_f64(inp.w[:, :inp.n] if inp.weight_kn else inp.w[:, :inp.k])
    if rows is not None:
        a = a[rows]
    return ogemm.gemm(a, w, not inp.weight_kn), ogemm.gemm(np.abs(a), np.abs(w), not inp.weight_kn)


def compare_gemm(c_gpu: torch.Tensor, ref: np.ndarray, absprod: np.ndarray, k: int,
                 rows=None, label: str = ""):
    """Element-wise bound for one bf16 rounding of an fp32 sum of K exact bf16
    products: |C - c| <= 2^-8 |c| + (1 + 2^-8) * 2 K 2^-24 * sum_k |a||b|
    (2 K u32 covers any summation order of K terms, with room for
    round-toward-zero additions inside the MFMA).  At least 97% of the elements
    must equal the exact product rounded to bf16."""
    g = c_gpu.float().cpu().double().numpy()
    if rows is not None:
        g = g[rows]
    assert np.isfinite(g).all(), f"{label}: non-finite GPU output"
    err = np.abs(g - ref)
    bound = 2.0**-8 * np.abs(ref) + (1 + 2.0**-8) * 2 * k * 2.0**-24 * absprod
    bad = err > bound
    exact = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    agree = float((g == exact).mean()) if g.size else 1.0
    ratio = float((err / np.maximum(bound, 1e-300)).max()) if g.size else 0.0
    note(f"{label}: max_err/bound={ratio:.3e} rounded-exact agreement={agree:.4f}")
    assert not bad.any(), f"{label}: {int(bad.sum())} elements beyond the bound"
    assert agree >= 0.97, f"{label}: only {agree:.4f} of elements equal the rounded exact value"
