"""Seeded synthetic inputs for the chunked flash-attention forward.

This module is shared by the fp64 oracle's tests, the GPU parity tests and the
benchmark.  It holds no attention arithmetic: it only draws random tensors,
builds sequence-length prefix sums, page tables and per-tensor fp8 codes.

Workload shapes (the five workloads of the method's pages, restated):
  * tiny causal GQA:      B=1, Hq=2,  Hkv=1, N=300,  D=64,  bf16
  * dense prefill:        B=1, Hq=Hkv=32,   N=8192, D=128, bf16
  * causal GQA varlen:    B=4, Hq=32, Hkv=8, lengths {4096, 2500, 1, 3969}, D=128
  * split-KV paged decode: 64 sequences x 1 token, Hq=32, Hkv=8, D=128,
                          context lengths uniform in [1, 32768], page size 16
  * fp8 wide-head prefill: B=1, Hq=Hkv=32, N=8192, D=192, e4m3 per-tensor scaled
  * batch-invariant GEMM: the per-rank tensor-parallel (TP4) layer shapes of an
    8B model that the method page times (M x K -> N): gate_up 4096 x 4096 ->
    6144, down 4096 x 3072 -> 4096, and the decode-sized M = 8 qkv (4096 ->
    1536) and gate_up (4096 -> 6144) products; bf16 N(0,1) activations and
    weights

All values are N(0,1) and unscaled (scaled fixtures hide corruption: ffpa-attn
PR "fp8 attention D=192" page, section "Tests / docs").  Tensors are produced on
the CPU with ``torch.Generator`` so that the same seed gives the same bytes on
every machine.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

E4M3_MAX = 448.0  # largest finite OCP E4M3FN value

TINY_CAUSAL = dict(name="tiny_causal_gqa", seqlens=[300], hq=2, hkv=1, d=64, causal=True)
DENSE_PREFILL = dict(name="dense_prefill", seqlens=[8192], hq=32, hkv=32, d=128, causal=False)
CAUSAL_VARLEN = dict(name="causal_gqa_varlen", seqlens=[4096, 2500, 1, 3969], hq=32, hkv=8, d=128,
                     causal=True)
PAGED_DECODE = dict(name="paged_decode", batch=64, hq=32, hkv=8, d=128, page_size=16,
                    ctx_min=1, ctx_max=32768, spare_pages=1024)
FP8_WIDE = dict(name="fp8_wide_head", seqlens=[8192], hq=32, hkv=32, d=192)
# One launch over a paged cache mixing the causal varlen prefill sequences,
# 512-token extends of prefixes that cross chunk boundaries, and decode steps
# (one query token) at short to maximal contexts; GQA 32/8, D=128.
MIXED_EXTEND = dict(name="mixed_paged_extend", hq=32, hkv=8, d=128, page_size=16, spare_pages=64,
                    ctx_lens=[4096, 2500, 3969, 8704, 8704, 16896, 16896, 1000, 9000, 20000,
                              32768],
                    q_lens=[4096, 2500, 3969, 512, 512, 512, 512, 1, 1, 1, 1])


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def cu_seqlens(lengths: Sequence[int]) -> torch.Tensor:
    """Exclusive prefix sum [0, l0, l0+l1, ...] as int32 (CPU)."""
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    assert out[-1] < 2**31
    return torch.from_numpy(out.astype(np.int32))


def randn_bf16(shape, gen: torch.Generator) -> torch.Tensor:
    """N(0,1) drawn in fp32 then rounded to bf16 (round-to-nearest-even)."""
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


@dataclasses.dataclass
class Fp8Tensor:
    """Per-tensor scaled OCP E4M3FN codes: value = decode(codes) * scale."""
    codes: torch.Tensor  # uint8, same shape as the source tensor
    scale: float         # fp32 dequantisation scale (amax / 448)


def quantize_e4m3(x: torch.Tensor) -> Fp8Tensor:
    """Per-tensor amax/448 scale, round-to-nearest-even into E4M3FN, saturating."""
    x = x.float()
    amax = float(x.abs().max())
    scale = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    y = (x / float(scale)).clamp(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return Fp8Tensor(codes=codes.contiguous(), scale=float(scale))


@dataclasses.dataclass
class PrefillInputs:
    q: torch.Tensor            # [total_q, Hq, D]  bf16 (or uint8 codes for fp8)
    k: torch.Tensor            # [total_k, Hkv, D]
    v: torch.Tensor            # [total_k, Hkv, D]
    cu_seqlens_q: torch.Tensor  # int32 [B+1]
    cu_seqlens_k: torch.Tensor  # int32 [B+1]
    seqlens_q: list
    seqlens_k: list
    hq: int
    hkv: int
    d: int
    scale: float
    causal: bool
    dtype: str = "bf16"
    q_scale: float = 1.0
    k_scale: float = 1.0
    v_scale: float = 1.0
    seed: int = 0


def prefill_inputs(seed: int, seqlens_q: Sequence[int], hq: int, hkv: int, d: int,
                   causal: bool, seqlens_k: Optional[Sequence[int]] = None,
                   dtype: str = "bf16", scale: Optional[float] = None) -> PrefillInputs:
    """Packed-varlen Q/K/V ~ N(0,1) for one prefill (or extend, when q_len < k_len) call."""
    seqlens_q = [int(x) for x in seqlens_q]
    seqlens_k = [int(x) for x in (seqlens_k if seqlens_k is not None else seqlens_q)]
    assert len(seqlens_q) == len(seqlens_k)
    tq, tk = sum(seqlens_q), sum(seqlens_k)
    g = _gen(seed)
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    if dtype == "bf16":
        q = randn_bf16((tq, hq, d), g)
        k = randn_bf16((tk, hkv, d), g)
        v = randn_bf16((tk, hkv, d), g)
        return PrefillInputs(q, k, v, cu_seqlens(seqlens_q), cu_seqlens(seqlens_k), seqlens_q,
                             seqlens_k, hq, hkv, d, float(scale), bool(causal), "bf16", seed=seed)
    if dtype == "fp8":
        qf = quantize_e4m3(torch.randn(tq, hq, d, generator=g))
        kf = quantize_e4m3(torch.randn(tk, hkv, d, generator=g))
        vf = quantize_e4m3(torch.randn(tk, hkv, d, generator=g))
        return PrefillInputs(qf.codes, kf.codes, vf.codes, cu_seqlens(seqlens_q),
                             cu_seqlens(seqlens_k), seqlens_q, seqlens_k, hq, hkv, d, float(scale),
                             bool(causal), "fp8", qf.scale, kf.scale, vf.scale, seed=seed)
    raise ValueError(dtype)


@dataclasses.dataclass
class DecodeInputs:
    q: torch.Tensor            # [B, Hq, D] bf16
    k_cache: torch.Tensor      # [num_pages, page_size, Hkv, D] bf16
    v_cache: torch.Tensor      # [num_pages, page_size, Hkv, D] bf16
    page_table: torch.Tensor   # int32 [B, max_pages_per_seq]
    context_lens: torch.Tensor  # int32 [B]
    hq: int
    hkv: int
    d: int
    page_size: int
    scale: float
    seed: int = 0
    dtype: str = "bf16"
    q_scale: float = 1.0
    k_scale: float = 1.0
    v_scale: float = 1.0


def decode_inputs(seed: int, batch: int, hq: int, hkv: int, d: int, page_size: int = 16,
                  context_lens: Optional[Sequence[int]] = None, ctx_min: int = 1,
                  ctx_max: int = 32768, spare_pages: int = 1024, poison: bool = True,
                  scale: Optional[float] = None, dtype: str = "bf16") -> DecodeInputs:
    """Paged KV cache with a seeded random page table.

    Live slots are N(0,1); slots past a sequence's context length and spare pages
    hold NaN when ``poison`` is set, so any read of a dead slot shows in the output.
    The table has ``ceil(max_ctx / page_size)`` columns; unused entries point at
    spare pages (or page 0 when there are none).
    """
    g = _gen(seed)
    if context_lens is None:
        ctx = torch.randint(ctx_min, ctx_max + 1, (batch,), generator=g, dtype=torch.int64)
    else:
        ctx = torch.tensor([int(c) for c in context_lens], dtype=torch.int64)
        assert len(ctx) == batch
    pages = [(int(c) + page_size - 1) // page_size for c in ctx]
    num_pages = sum(pages) + spare_pages
    max_pages = max(1, max(pages) if pages else 1)
    perm = torch.randperm(num_pages, generator=g)
    table = torch.empty(batch, max_pages, dtype=torch.int32)
    pos = 0
    filler = perm[sum(pages):] if spare_pages > 0 else torch.zeros(1, dtype=torch.int64)
    for b in range(batch):
        n = pages[b]
        table[b, :n] = perm[pos:pos + n].to(torch.int32)
        pos += n
        rest = max_pages - n
        if rest > 0:
            table[b, n:] = filler[torch.arange(rest) % len(filler)].to(torch.int32)
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    q32 = torch.randn(batch, hq, d, generator=g)
    k32 = torch.randn(num_pages, page_size, hkv, d, generator=g)
    v32 = torch.randn(num_pages, page_size, hkv, d, generator=g)
    if poison:
        live = torch.zeros(num_pages, page_size, dtype=torch.bool)
        for b in range(batch):
            c = int(ctx[b])
            for j in range(pages[b]):
                p = int(table[b, j])
                live[p, : min(page_size, c - j * page_size)] = True
        k32[~live] = float("nan")
        v32[~live] = float("nan")
    if dtype == "bf16":
        return DecodeInputs(q32.to(torch.bfloat16), k32.to(torch.bfloat16), v32.to(torch.bfloat16),
                            table, ctx.to(torch.int32), hq, hkv, d, page_size, float(scale), seed)
    if dtype == "fp8":
        qf = quantize_e4m3(q32)
        kf = quantize_e4m3(torch.nan_to_num(k32, nan=0.0))
        vf = quantize_e4m3(torch.nan_to_num(v32, nan=0.0))
        kc, vc = kf.codes.clone(), vf.codes.clone()
        if poison:
            kc[~live] = 0x7F  # E4M3FN NaN code
            vc[~live] = 0x7F
        return DecodeInputs(qf.codes, kc, vc, table, ctx.to(torch.int32), hq, hkv, d, page_size,
                            float(scale), seed, "fp8", qf.scale, kf.scale, vf.scale)
    raise ValueError(dtype)


@dataclasses.dataclass
class ExtendInputs:
    """A mixed prefill / extend / decode batch over a paged KV cache.

    Sequence b has ctx_lens[b] tokens and q_lens[b] query rows, its last
    q_lens[b] tokens.  ``q_full``/``k``/``v`` hold every token of every sequence
    packed contiguously (``cu_full``), ``q`` the query rows only (``cu_seqlens_q``),
    and the caches the same K/V tokens placed in pages by a seeded random table."""
    q: torch.Tensor             # [sum(q_lens), Hq, D]
    cu_seqlens_q: torch.Tensor  # int32 [B+1]
    q_full: Optional[torch.Tensor]  # [sum(ctx_lens), Hq, D] (with full_q) or None
    k: torch.Tensor             # [sum(ctx_lens), Hkv, D]
    v: torch.Tensor
    cu_full: torch.Tensor       # int32 [B+1] over ctx_lens
    k_cache: torch.Tensor       # [num_pages, page_size, Hkv, D]
    v_cache: torch.Tensor
    page_table: torch.Tensor    # int32 [B, max_pages]
    context_lens: torch.Tensor  # int32 [B]
    q_lens: list
    ctx_lens: list
    hq: int
    hkv: int
    d: int
    page_size: int
    scale: float
    causal: bool
    dtype: str = "bf16"
    q_scale: float = 1.0
    k_scale: float = 1.0
    v_scale: float = 1.0
    seed: int = 0


def extend_inputs(seed: int, ctx_lens: Sequence[int], q_lens: Sequence[int], hq: int, hkv: int,
                  d: int, causal: bool = True, page_size: int = 16, spare_pages: int = 8,
                  poison: bool = True, dtype: str = "bf16", scale: Optional[float] = None,
                  full_q: bool = False) -> ExtendInputs:
    """K/V ~ N(0,1) for every token, Q ~ N(0,1) for the query rows of each
    sequence's tail (for every token with ``full_q``), and a paged copy of K/V
    (dead slots and spare pages NaN when ``poison``)."""
    ctx_lens = [int(x) for x in ctx_lens]
    q_lens = [int(x) for x in q_lens]
    assert len(ctx_lens) == len(q_lens) and all(0 <= a <= b for a, b in zip(q_lens, ctx_lens))
    g = _gen(seed)
    tk = sum(ctx_lens)
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    q32 = torch.randn(tk if full_q else sum(q_lens), hq, d, generator=g)
    k32 = torch.randn(tk, hkv, d, generator=g)
    v32 = torch.randn(tk, hkv, d, generator=g)
    pages = [(c + page_size - 1) // page_size for c in ctx_lens]
    num_pages = sum(pages) + spare_pages
    max_pages = max(1, max(pages) if pages else 1)
    perm = torch.randperm(num_pages, generator=g)
    table = torch.zeros(len(ctx_lens), max_pages, dtype=torch.int32)
    pos = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[pos:pos + n].to(torch.int32)
        pos += n
        if n < max_pages:  # unused entries point at spare pages (or page 0)
            spare = perm[sum(pages):] if spare_pages > 0 else torch.zeros(1, dtype=torch.int64)
            table[b, n:] = spare[torch.arange(max_pages - n) % len(spare)].to(torch.int32)
    if dtype == "bf16":
        qf, kf, vf = q32.to(torch.bfloat16), k32.to(torch.bfloat16), v32.to(torch.bfloat16)
        qs = ks = vs = 1.0
        dead = torch.tensor(float("nan")).to(torch.bfloat16)
        zero_cache = torch.zeros(num_pages, page_size, hkv, d, dtype=torch.bfloat16)
    elif dtype == "fp8":
        fq, fk, fv = quantize_e4m3(q32), quantize_e4m3(k32), quantize_e4m3(v32)
        qf, kf, vf = fq.codes, fk.codes, fv.codes
        qs, ks, vs = fq.scale, fk.scale, fv.scale
        dead = torch.tensor(0x7F, dtype=torch.uint8)  # E4M3FN NaN code
        zero_cache = torch.zeros(num_pages, page_size, hkv, d, dtype=torch.uint8)
    else:
        raise ValueError(dtype)
    kc, vc = zero_cache.clone(), zero_cache.clone()
    if poison:
        kc[:] = dead
        vc[:] = dead
    cu = cu_seqlens(ctx_lens)
    rows = []
    for b, c in enumerate(ctx_lens):
        s0 = int(cu[b])
        j = torch.arange(c)
        pg = table[b, (j // page_size)].long()
        kc[pg, j % page_size] = kf[s0:s0 + c]
        vc[pg, j % page_size] = vf[s0:s0 + c]
        rows.append(torch.arange(s0 + c - q_lens[b], s0 + c))
    idx = torch.cat(rows) if rows else torch.zeros(0, dtype=torch.int64)
    q_rows = qf[idx].contiguous() if full_q else qf
    return ExtendInputs(q_rows, cu_seqlens(q_lens), qf if full_q else None, kf, vf, cu, kc, vc,
                        table,
                        torch.tensor(ctx_lens, dtype=torch.int32), q_lens, ctx_lens, hq, hkv, d,
                        page_size, float(scale), bool(causal), dtype, qs, ks, vs, seed)


# (name, M, N, K): C[M, N] = A[M, K] W^T with W [N, K]
GEMM_SHAPES = [("gate_up", 4096, 6144, 4096), ("down", 4096, 4096, 3072),
               ("qkv_decode", 8, 1536, 4096), ("gate_up_decode", 8, 6144, 4096)]


@dataclasses.dataclass
class GemmInputs:
    a: torch.Tensor        # bf16 [M, lda] (rows of length K inside)
    w: torch.Tensor        # bf16 [N, ldw] ([N, K] layout) or [K, ldw] ([K, N] layout)
    m: int
    n: int
    k: int
    weight_kn: bool
    seed: int


def gemm_inputs(seed: int, m: int, n: int, k: int, weight_kn: bool = False, pad_a: int = 0,
                pad_w: int = 0, poison: bool = False) -> GemmInputs:
    """N(0,1) bf16 operands.  pad_a / pad_w widen the row strides (lda = K + pad_a,
    ldw = K or N + pad_w); with poison the padding holds NaN, which must never
    reach a valid output."""
    g = _gen(seed)
    a = randn_bf16((m, k), g)
    w = randn_bf16((k, n) if weight_kn else (n, k), g)
    fill = float("nan") if poison else 0.0
    if pad_a:
        a = torch.cat([a, torch.full((m, pad_a), fill, dtype=torch.bfloat16)], dim=1)
    if pad_w:
        w = torch.cat([w, torch.full((w.shape[0], pad_w), fill, dtype=torch.bfloat16)], dim=1)
    return GemmInputs(a, w, m, n, k, weight_kn, seed)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16/fp32 CPU tensor to a float64 NumPy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def workload_prefill(cfg: dict, seed: int, dtype: str = "bf16", causal: Optional[bool] = None):
    c = cfg["causal"] if causal is None else causal
    return prefill_inputs(seed, cfg["seqlens"], cfg["hq"], cfg["hkv"], cfg["d"], c, dtype=dtype)
