"""Pins for the fp64 GEMM oracle, checked against things other than itself.

The operation is the batch-invariant GEMM of the RL-Kernel page "MFMA
batch-invariant GEMM and chunked Triton attention", section 1: C = A W^T for an
[N, K] weight (or A B for a [K, N] one), K consumed in 64-wide blocks inside
1024-wide chunks.  The page prints no worked example, so the pins are brute
force on tiny inputs, integer closed forms, special cases and invariants; the
``test_planted_*`` tests inject plausible slips (a dropped ragged chunk, a
transposed weight, a chunk partial that is not reset) into the oracle on the
CPU and check that a pin catches each.
"""
import numpy as np
import pytest

import oracle.gemm as og

RNG = np.random.default_rng(4321)


def brute_force(a, w, weight_nk=True):
    """Triple loop: C[i][j] = sum_k A[i][k] * B[k][j] with B = W^T for [N, K]."""
    m, k = len(a), len(a[0])
    n = len(w) if weight_nk else len(w[0])
    out = [[0.0] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            s = 0.0
            for t in range(k):
                s += float(a[i][t]) * float(w[j][t] if weight_nk else w[t][j])
            out[i][j] = s
    return np.array(out)


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (3, 5, 7), (3, 7, 7), (4, 3, 70), (2, 6, 130)])
@pytest.mark.parametrize("weight_nk", [True, False])
def test_gemm_matches_brute_force(m, n, k, weight_nk):
    a = RNG.standard_normal((m, k))
    w = RNG.standard_normal((n, k) if weight_nk else (k, n))
    ref = brute_force(a.tolist(), w.tolist(), weight_nk)
    np.testing.assert_allclose(og.gemm(a, w, weight_nk), ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(og.gemm_chunked(a, w, weight_nk), ref, rtol=1e-12, atol=1e-12)


def _closed_form(m, n, k):
    """A[i][t] = i + t, W[j][t] = j - 2t: C[i][j] = sum_t (i + t)(j - 2t)
    = K i j + (j - 2 i) S1 - 2 S2 with S1 = sum t, S2 = sum t^2 over t < K."""
    s1 = k * (k - 1) // 2
    s2 = (k - 1) * k * (2 * k - 1) // 6
    i = np.arange(m)[:, None]
    j = np.arange(n)[None, :]
    return k * i * j + (j - 2 * i) * s1 - 2 * s2


@pytest.mark.parametrize("k", [1, 64, 1000, 1024, 2500])
def test_integer_closed_form(k):
    m, n = 6, 9
    a = (np.arange(m)[:, None] + np.arange(k)[None, :]).astype(np.float64)
    w = (np.arange(n)[:, None] - 2 * np.arange(k)[None, :]).astype(np.float64)
    want = _closed_form(m, n, k).astype(np.float64)  # exact: every value is below 2^53
    assert np.array_equal(og.gemm(a, w), want)
    assert np.array_equal(og.gemm_chunked(a, w), want)
    assert np.array_equal(og.gemm(a, w.T.copy(), weight_nk=False), want)
    assert np.array_equal(og.gemm_chunked(a, w.T.copy(), weight_nk=False), want)


@pytest.mark.parametrize("k", [1, 63, 64, 65, 1023, 1024, 1025, 1100, 2500, 4096])
def test_chunked_equals_plain(k):
    a = RNG.standard_normal((5, k))
    w = RNG.standard_normal((7, k))
    scale = np.abs(a) @ np.abs(w).T
    err = np.abs(og.gemm_chunked(a, w) - og.gemm(a, w))
    assert (err <= 4 * k * 2.0**-53 * scale).all()


def test_identity_and_layouts():
    k = 96
    w = RNG.standard_normal((40, k))
    # A = I_K picks out the weight: C = W^T for an [N, K] weight.
    assert np.array_equal(og.gemm(np.eye(k), w), w.T)
    assert np.array_equal(og.gemm_chunked(np.eye(k), w), w.T)
    # the [K, N] layout of the same weight gives the same product
    a = RNG.standard_normal((9, k))
    np.testing.assert_allclose(og.gemm(a, w.T.copy(), weight_nk=False), og.gemm(a, w),
                               rtol=1e-13, atol=1e-13)


def test_rows_are_independent():
    """Row i of C depends only on row i of A: a row subset gives the same rows."""
    a = RNG.standard_normal((33, 1100))
    w = RNG.standard_normal((12, 1100))
    full = og.gemm_chunked(a, w)
    rows = [0, 5, 17, 32]
    np.testing.assert_allclose(og.gemm_chunked(a[rows], w), full[rows], rtol=1e-13, atol=1e-12)


def test_rank_one_closed_form():
    """A = u x^T, W = v y^T: C = (x . y) u v^T."""
    u, v = RNG.standard_normal(7), RNG.standard_normal(5)
    x, y = RNG.standard_normal(1500), RNG.standard_normal(1500)
    c = og.gemm_chunked(np.outer(u, x), np.outer(v, y))
    np.testing.assert_allclose(c, float(x @ y) * np.outer(u, v), rtol=1e-10, atol=1e-10)


def test_flop_count():
    m, n, k = 3, 4, 5
    count = 0
    for _ in range(m * n):
        for _ in range(k):
            count += 2  # one multiply, one add
    assert og.gemm_flops(m, n, k) == count
    assert og.gemm_flops(4096, 6144, 4096) == 2 * 4096 * 6144 * 4096


# ---------------------------------------------------------------------------
# Planted mistakes: each slip is injected into the oracle on the CPU and at
# least one pin above must fail on it.
# ---------------------------------------------------------------------------
def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_dropped_ragged_chunk(monkeypatch):
    def chunked_drop(a, w, weight_nk=True):
        a, b = og._operands(a, w, weight_nk)
        m, k = a.shape
        total = np.zeros((m, b.shape[1]))
        for c0 in range(0, k - og.CHUNK_K + 1, og.CHUNK_K):  # misses a partial last chunk
            part = np.zeros_like(total)
            for k0 in range(c0, c0 + og.CHUNK_K, og.BLOCK_K):
                part = part + a[:, k0:k0 + og.BLOCK_K] @ b[k0:k0 + og.BLOCK_K, :]
            total = total + part
        return total
    monkeypatch.setattr(og, "gemm_chunked", chunked_drop)
    assert _fails(lambda: test_chunked_equals_plain(2500))
    assert _fails(lambda: test_integer_closed_form(1000))


def test_planted_transposed_weight(monkeypatch):
    real = og._operands

    def swapped(a, w, weight_nk):
        return real(a, w, not weight_nk)
    monkeypatch.setattr(og, "_operands", swapped)
    assert _fails(lambda: test_gemm_matches_brute_force(3, 7, 7, True))  # square: no shape error


def test_planted_partial_not_reset(monkeypatch):
    def carried(a, w, weight_nk=True):
        a, b = og._operands(a, w, weight_nk)
        m, k = a.shape
        total = np.zeros((m, b.shape[1]))
        part = np.zeros_like(total)
        for c0 in range(0, k, og.CHUNK_K):
            for k0 in range(c0, min(c0 + og.CHUNK_K, k), og.BLOCK_K):
                part = part + a[:, k0:k0 + og.BLOCK_K] @ b[k0:k0 + og.BLOCK_K, :]
            total = total + part  # earlier chunks counted again
        return total
    monkeypatch.setattr(og, "gemm_chunked", carried)
    assert _fails(lambda: test_integer_closed_form(2500))
