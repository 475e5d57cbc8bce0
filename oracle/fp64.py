"""fp64 CPU oracle for the batch-invariant chunked flash-attention forward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's ``smoke()`` check and the
benchmark's ``cpu_baseline`` leg may import this module.  It shares no code with
the HIP path: it reads plain NumPy arrays holding the *stored* input values
(bf16 widened exactly to fp64, E4M3FN codes decoded here from the format
definition and multiplied by their per-tensor scale in fp64) and returns fp64.

What it computes (RL-Kernel PR "MFMA batch-invariant GEMM and chunked Triton
attention" page, section 2 "Chunked-KV Triton flash attention"): the attention
forward ``O = softmax(scale * Q K^T + mask) V`` for full-sequence forward,
prefill, prefix-cached extend and single-token paged decode.

Readings of points the page leaves open (each restated in the design notes):
  * the mask is a key-length bound plus an optional causal bound, aligned to the
    bottom-right corner: key j is visible from query row i of a sequence with
    L_q queries and L_k keys iff ``j < L_k and (not causal or j <= i + L_k - L_q)``;
    this is the only alignment under which a decode row equals the last prefill
    row, which the page requires;
  * a sliding window (local attention; window-sized bounds, aiter MQA-logits
    page) ``(w_left, w_right)``, -1 meaning unbounded on that side, adds
    ``j >= i + L_k - L_q - w_left`` and ``j <= i + L_k - L_q + w_right`` on the
    same bottom-right diagonal;
  * grouped-query attention maps query head h to key/value head
    ``h // (Hq // Hkv)`` (contiguous groups);
  * a row with no visible key returns O = 0 and lse = -inf;
  * lse is the natural-log sum of exp(scale * q.k) over the visible keys.

Two evaluations are given:
  ``attention``          the plain definition, one (sequence, head) at a time,
                         row-max-subtracted softmax and two matrix products;
  ``attention_chunked``  the method's own steps in real (fp64) arithmetic:
                         64-key blocks inside 512-key chunks, each chunk's
                         online softmax from an empty state, chunks merged in
                         ascending order with the exact max/sum rescale, and
                         fully masked blocks leaving a row untouched.  The two
                         agree to rounding because the rescale is an identity;
                         the tests check that, which pins the algorithm.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

BLOCK_KEYS = 64    # keys per online-softmax update (method page, section 2)
CHUNK_KEYS = 512   # keys per chunk, each starting from an empty state (same section)
_ROW_BLOCK = 1024  # rows evaluated together by the plain oracle (rows are independent)


# ----------------------------------------------------------------------------
# E4M3FN decoding (OCP 8-bit floating point specification, E4M3 format):
# 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
# subnormal (m/8 * 2^-6); S.1111.111 is NaN; there are no infinities.
# ----------------------------------------------------------------------------
def e4m3fn_table() -> np.ndarray:
    """The 256 fp64 values of the E4M3FN codes, decoded field by field."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            out[code] = math.nan
        elif exp == 0:
            out[code] = sign * (man / 8.0) * 2.0 ** -6
        else:
            out[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
    return out


_E4M3 = e4m3fn_table()


def dequantize_e4m3(codes: np.ndarray, scale: float) -> np.ndarray:
    """fp64 value of per-tensor scaled E4M3FN codes: decode(code) * scale."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)] * np.float64(scale)


# ----------------------------------------------------------------------------
# Mask (reading of "+ mask"; see module docstring)
# ----------------------------------------------------------------------------
def visible(rows: np.ndarray, lq: int, lk: int, causal: bool,
            window: Sequence[int] = (-1, -1)) -> np.ndarray:
    """Boolean [len(rows), lk]: key j visible from local query row i."""
    j = np.arange(lk)[None, :]
    diag = np.asarray(rows)[:, None] + (lk - lq)  # the row's own position among the keys
    ok = j < lk
    if causal:
        ok = ok & (j <= diag)
    wl, wr = int(window[0]), int(window[1])
    if wl >= 0:
        ok = ok & (j >= diag - wl)
    if wr >= 0:
        ok = ok & (j <= diag + wr)
    return np.broadcast_to(ok, (len(rows), lk)).copy()


def _check(q, k, v, cu_q, cu_k, hq, hkv):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    assert q.ndim == 3 and k.ndim == 3 and v.shape == k.shape
    assert q.shape[1] == hq and k.shape[1] == hkv and hq % hkv == 0
    assert len(cu_q) == len(cu_k) and cu_q[-1] <= q.shape[0] and cu_k[-1] <= k.shape[0]
    return q, k, v, cu_q, cu_k


# ----------------------------------------------------------------------------
# Plain definition
# ----------------------------------------------------------------------------
def attention(q, k, v, cu_seqlens_q, cu_seqlens_k, hq: int, hkv: int, scale: float,
              causal: bool, rows: Optional[Sequence[int]] = None,
              window: Sequence[int] = (-1, -1)):
    """O = softmax(scale * Q K^T + mask) V for packed variable-length sequences.

    q: [total_q, Hq, D], k/v: [total_k, Hkv, D] (fp64 values of the stored inputs);
    cu_seqlens_*: [B+1] prefix sums.  Returns (O [total_q, Hq, D], lse [total_q, Hq])
    in fp64.  With ``rows`` (global query-row indices) only those rows are
    evaluated; the other rows of the result are NaN.
    Follows the method page, section 2 (the softmax-attention forward it serves
    for every caller).
    """
    q, k, v, cu_q, cu_k = _check(q, k, v, cu_seqlens_q, cu_seqlens_k, hq, hkv)
    total_q, _, d = q.shape
    group = hq // hkv
    out = np.full((total_q, hq, d), np.nan)
    lse = np.full((total_q, hq), np.nan)
    want = None if rows is None else np.zeros(total_q, dtype=bool)
    if want is not None:
        want[np.asarray(rows, dtype=np.int64)] = True
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        lq, lk = q1 - q0, k1 - k0
        local = np.arange(lq) if want is None else np.nonzero(want[q0:q1])[0]
        for r0 in range(0, len(local), _ROW_BLOCK):
            rl = local[r0:r0 + _ROW_BLOCK]
            if len(rl) == 0:
                continue
            mask = visible(rl, lq, lk, causal, window)
            has_key = mask.any(axis=1)
            for h in range(hq):
                g = h // group
                kb, vb = k[k0:k1, g, :], v[k0:k1, g, :]
                s = scale * (q[q0 + rl, h, :] @ kb.T)
                s = np.where(mask, s, -np.inf)
                mx = np.where(has_key, s.max(axis=1, initial=-np.inf), 0.0)
                e = np.where(mask, np.exp(s - mx[:, None]), 0.0)
                l = e.sum(axis=1)
                o = np.zeros((len(rl), d))
                o[has_key] = (e[has_key] @ vb) / l[has_key, None]
                out[q0 + rl, h, :] = o
                lse[q0 + rl, h] = np.where(has_key, mx + np.log(np.where(has_key, l, 1.0)), -np.inf)
    return out, lse


# ----------------------------------------------------------------------------
# The method's steps in fp64 (self-check of the algorithm, not of GPU bits)
# ----------------------------------------------------------------------------
def _block_update(state, s, vb):
    """One 64-key online-softmax update from the method page, section 2.

    state = (m, l, acc) per row; s: [rows, keys] scaled scores with -inf where
    masked; vb: [keys, D].  Rows whose block is fully masked keep their state.
    """
    m, l, acc = state
    mblk = s.max(axis=1, initial=-np.inf)
    live = mblk > -np.inf
    if not live.any():
        return state
    m_new = np.where(live, np.maximum(m, mblk), m)
    with np.errstate(invalid="ignore"):
        alpha = np.where(live & (m > -np.inf), np.exp(m - m_new), 0.0)
        p = np.where(live[:, None], np.exp(s - np.where(live, m_new, 0.0)[:, None]), 0.0)
    l_new = np.where(live, l * alpha + p.sum(axis=1), l)
    acc_new = np.where(live[:, None], acc * alpha[:, None] + p @ vb, acc)
    return m_new, l_new, acc_new


def _merge(total, part):
    """Fold one chunk partial into the running state: the exact max/sum rescale."""
    M, L, A = total
    m, l, acc = part
    live = m > -np.inf
    first = live & ~(M > -np.inf)
    both = live & (M > -np.inf)
    Mn = np.where(live, np.maximum(M, m), M)
    with np.errstate(invalid="ignore"):
        a = np.where(both, np.exp(M - Mn), 1.0)
        bcoef = np.where(both, np.exp(m - Mn), 1.0)
    Ln = np.where(first, l, np.where(both, L * a + l * bcoef, L))
    An = np.where(first[:, None], acc, np.where(both[:, None], A * a[:, None] + acc * bcoef[:, None], A))
    return Mn, Ln, An


def chunk_partials(qrows, kb, vb, rows_local, lq, lk, scale, causal, window=(-1, -1)):
    """Per-chunk partial states (m_c, l_c, acc_c) for the given rows of one head.

    Each chunk c covers absolute keys [512c, 512c+512) and folds its 64-key blocks
    in ascending order from the empty state (-inf, 0, 0).  Returns a list over c.
    """
    n = len(rows_local)
    d = vb.shape[1]
    mask = visible(rows_local, lq, lk, causal, window)
    parts = []
    for c0 in range(0, lk, CHUNK_KEYS):
        st = (np.full(n, -np.inf), np.zeros(n), np.zeros((n, d)))
        for b0 in range(c0, min(c0 + CHUNK_KEYS, lk), BLOCK_KEYS):
            b1 = min(b0 + BLOCK_KEYS, lk)
            s = scale * (qrows @ kb[b0:b1].T)
            s = np.where(mask[:, b0:b1], s, -np.inf)
            st = _block_update(st, s, vb[b0:b1])
        parts.append(st)
    return parts


def attention_chunked(q, k, v, cu_seqlens_q, cu_seqlens_k, hq: int, hkv: int, scale: float,
                      causal: bool, window: Sequence[int] = (-1, -1)):
    """The chunked evaluation: partials per 512-key chunk, merged ascending, then
    O = A / L (0 for a row with no visible key) and lse = M + log L."""
    q, k, v, cu_q, cu_k = _check(q, k, v, cu_seqlens_q, cu_seqlens_k, hq, hkv)
    total_q, _, d = q.shape
    group = hq // hkv
    out = np.zeros((total_q, hq, d))
    lse = np.full((total_q, hq), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        lq, lk = q1 - q0, k1 - k0
        rl = np.arange(lq)
        if lq == 0:
            continue
        for h in range(hq):
            g = h // group
            parts = chunk_partials(q[q0:q1, h, :], k[k0:k1, g, :], v[k0:k1, g, :], rl, lq, lk,
                                   scale, causal, window)
            tot = (np.full(lq, -np.inf), np.zeros(lq), np.zeros((lq, d)))
            for p in parts:
                tot = _merge(tot, p)
            M, L, A = tot
            ok = L > 0
            out[q0:q1, h, :][ok] = A[ok] / L[ok, None]
            lse[q0:q1, h] = np.where(ok, M + np.log(np.where(ok, L, 1.0)), -np.inf)
    return out, lse


# ----------------------------------------------------------------------------
# Paged decode: one query token per sequence over a paged KV cache
# ----------------------------------------------------------------------------
def gather_pages(cache, page_table_row, ctx: int, page_size: int):
    """Contiguous [ctx, Hkv, D] view of one sequence's keys (or values):
    token j lives in page ``page_table_row[j // page_size]`` at slot ``j % page_size``."""
    j = np.arange(ctx)
    pages = np.asarray(page_table_row, dtype=np.int64)[j // page_size]
    return np.asarray(cache)[pages, j % page_size]


def paged_decode(q, k_cache, v_cache, page_table, context_lens, hq: int, hkv: int,
                 scale: float, page_size: int, window_left: int = -1):
    """Single-token decode: for sequence b the query is the last row of a
    sequence of length ctx_b, so every cached key j < ctx_b is visible (with a
    left window w, keys j >= ctx_b - 1 - w).

    q: [B, Hq, D]; caches: [pages, page_size, Hkv, D]; page_table: [B, max_pages].
    Returns (O [B, Hq, D], lse [B, Hq]) in fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    bsz, _, d = q.shape
    out = np.zeros((bsz, hq, d))
    lse = np.full((bsz, hq), -np.inf)
    for b in range(bsz):
        ctx = int(context_lens[b])
        kb = gather_pages(k_cache, page_table[b], ctx, page_size).astype(np.float64)
        vb = gather_pages(v_cache, page_table[b], ctx, page_size).astype(np.float64)
        o, l = attention(q[b:b + 1], kb, vb, [0, 1], [0, ctx], hq, hkv, scale, causal=True,
                         window=(window_left, -1))
        out[b], lse[b] = o[0], l[0]
    return out, lse


def attention_flops(seqlens_q, seqlens_k, hq: int, d: int, causal: bool,
                    window: Sequence[int] = (-1, -1)) -> int:
    """Algorithmic FLOP count: 4*D per visible (query, key) pair per query head
    (2*D for q.k and 2*D for p*v).  Chunking adds no counted work."""
    total = 0
    wl, wr = int(window[0]), int(window[1])
    for lq, lk in zip(seqlens_q, seqlens_k):
        lq, lk = int(lq), int(lk)
        if wl < 0 and wr < 0:
            total += _causal_pairs(lq, lk) if causal else lq * lk
        else:
            total += _window_pairs(lq, lk, causal, wl, wr)
    return 4 * d * hq * total


def _window_pairs(lq: int, lk: int, causal: bool, wl: int, wr: int) -> int:
    # per row i the visible keys form [max(0, i+off-wl), min(lk, i+off+1 or i+off+wr+1, lk))
    off = lk - lq
    i = np.arange(lq, dtype=np.int64)
    lo = np.clip(i + off - wl, 0, lk) if wl >= 0 else np.zeros(lq, dtype=np.int64)
    hi = np.full(lq, lk, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, np.clip(i + off + 1, 0, lk))
    if wr >= 0:
        hi = np.minimum(hi, np.clip(i + off + wr + 1, 0, lk))
    return int(np.maximum(hi - lo, 0).sum())


def _causal_pairs(lq: int, lk: int) -> int:
    # sum over i in [0, lq) of clamp(i + lk - lq + 1, 0, lk)
    off = lk - lq
    i = np.arange(lq, dtype=np.int64)
    return int(np.clip(i + off + 1, 0, lk).sum())
