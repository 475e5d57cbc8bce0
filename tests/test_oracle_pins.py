"""Pins for the fp64 oracle, checked against things other than itself.

Each pin is chosen so that a plausible slip in the oracle (a dropped scale, a
wrong causal offset, a transposed operand, a merge without rescale, a wrong
GQA map, a wrong E4M3 field) fails at least one of them; ``test_planted_*``
plant such slips into the oracle on the CPU and check that a pin catches each.

The definition being pinned is the attention forward served by the chunked
kernel on the RL-Kernel "MFMA batch-invariant GEMM and chunked Triton
attention" page, section 2.  No page prints a worked attention example, so the
pins are brute force, closed forms and invariants.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.fp64 as oatt

RNG = np.random.default_rng(1234)


def brute_force(q, k, v, cu_q, cu_k, hq, hkv, scale, causal, window=(-1, -1)):
    """Textbook softmax attention with explicit Python loops and math.exp.
    window = (w_left, w_right), -1 unbounded: key j in [diag - w_left, diag + w_right]
    around the row's bottom-right diagonal position diag = i + L_k - L_q."""
    tq, _, d = q.shape
    out = [[[0.0] * d for _ in range(hq)] for _ in range(tq)]
    lse = [[-math.inf] * hq for _ in range(tq)]
    grp = hq // hkv
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        lq, lk = q1 - q0, k1 - k0
        for h in range(hq):
            g = h // grp
            for i in range(lq):
                diag = i + lk - lq
                keys = [j for j in range(lk)
                        if ((not causal) or j <= diag)
                        and (window[0] < 0 or j >= diag - window[0])
                        and (window[1] < 0 or j <= diag + window[1])]
                if not keys:
                    continue
                s = []
                for j in keys:
                    dot = 0.0
                    for t in range(d):
                        dot += float(q[q0 + i, h, t]) * float(k[k0 + j, g, t])
                    s.append(scale * dot)
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                z = sum(w)
                for t in range(d):
                    out[q0 + i][h][t] = sum(w[n] * float(v[k0 + j, g, t]) for n, j in enumerate(keys)) / z
                lse[q0 + i][h] = mx + math.log(z)
    return np.array(out, dtype=np.float64).reshape(tq, hq, d), np.array(lse).reshape(tq, hq)


def make(seqlens_q, seqlens_k, hq, hkv, d, seed=0, scale_v=1.0):
    rng = np.random.default_rng(seed)
    tq, tk = sum(seqlens_q), sum(seqlens_k)
    q = rng.standard_normal((tq, hq, d))
    k = rng.standard_normal((tk, hkv, d))
    v = rng.standard_normal((tk, hkv, d)) * scale_v
    cu_q = np.concatenate([[0], np.cumsum(seqlens_q)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(seqlens_k)]).astype(np.int64)
    return q, k, v, cu_q, cu_k


SMALL_CASES = [
    # (seqlens_q, seqlens_k, hq, hkv, d, causal)
    ([7], [7], 2, 1, 5, True),
    ([7], [7], 2, 2, 4, False),
    ([3, 9, 1], [3, 9, 1], 4, 2, 3, True),
    ([2, 5], [6, 11], 2, 1, 4, True),      # extend: q_len < k_len, bottom-right aligned
    ([6, 3], [4, 3], 2, 1, 3, True),       # q_len > k_len: leading rows see no key
    ([4, 0, 5], [4, 0, 5], 3, 1, 2, False),  # an empty sequence in the batch
    ([5], [0], 1, 1, 3, False),            # zero keys
]


@pytest.mark.parametrize("case", SMALL_CASES)
def test_plain_matches_brute_force(case):
    sq, sk, hq, hkv, d, causal = case
    q, k, v, cu_q, cu_k = make(sq, sk, hq, hkv, d, seed=len(sq) * 7 + d)
    scale = 0.37
    o, l = oracle.attention(q, k, v, cu_q, cu_k, hq, hkv, scale, causal)
    ob, lb = brute_force(q, k, v, cu_q, cu_k, hq, hkv, scale, causal)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(l), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(l[fin], lb[fin], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lens", [([1300], [1300]), ([70, 700], [600, 1100]), ([513, 64], [513, 64])])
def test_chunked_equals_plain(causal, lens):
    """The chunked evaluation (64-key blocks in 512-key chunks, ascending exact
    rescale) equals the plain definition up to fp64 rounding: the rescale is an
    algebraic identity, so this pins the algorithm's steps."""
    sq, sk = lens
    q, k, v, cu_q, cu_k = make(sq, sk, 4, 2, 8, seed=sum(sq))
    o1, l1 = oracle.attention(q, k, v, cu_q, cu_k, 4, 2, 1 / math.sqrt(8), causal)
    o2, l2 = oracle.attention_chunked(q, k, v, cu_q, cu_k, 4, 2, 1 / math.sqrt(8), causal)
    np.testing.assert_allclose(o2, o1, rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(l1), np.isneginf(l2))
    fin = np.isfinite(l1)
    np.testing.assert_allclose(l2[fin], l1[fin], rtol=1e-12, atol=1e-12)


def test_chunk_partials_start_empty_and_cover_absolute_keys():
    """Chunk c's partial only sees keys [512c, 512c+512): with V one-hot on the
    chunk index, acc_c / l_c is exactly the indicator of chunk c."""
    lk, d = 1500, 4
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, d))
    k = rng.standard_normal((lk, d))
    v = np.zeros((lk, 3))
    v[np.arange(lk), np.arange(lk) // 512] = 1.0
    parts = oatt.chunk_partials(q, k, v, np.array([0]), 1, lk, 0.5, False)
    assert len(parts) == 3
    for c, (m, l, acc) in enumerate(parts):
        expect = np.zeros(3)
        expect[c] = 1.0
        np.testing.assert_allclose(acc[0] / l[0], expect, atol=1e-15)
        # m_c is the max of the chunk's own scores
        assert m[0] == pytest.approx(np.max(0.5 * (k[512 * c:512 * (c + 1)] @ q[0])), rel=1e-15)


def test_rows_sum_to_one():
    q, k, v, cu_q, cu_k = make([300, 45], [300, 45], 2, 1, 6, seed=5)
    for causal in (False, True):
        o, _ = oracle.attention(q, k, np.ones_like(v), cu_q, cu_k, 2, 1, 0.8, causal)
        np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-13)
        o, _ = oracle.attention_chunked(q, k, np.ones_like(v), cu_q, cu_k, 2, 1, 0.8, causal)
        np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-13)


def test_key_permutation_invariance_dense():
    q, k, v, cu_q, cu_k = make([40], [700], 2, 2, 5, seed=9)
    perm = RNG.permutation(700)
    o1, l1 = oracle.attention(q, k, v, cu_q, cu_k, 2, 2, 0.5, False)
    o2, l2 = oracle.attention(q, k[perm], v[perm], cu_q, cu_k, 2, 2, 0.5, False)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-13)


def test_all_masked_rows():
    # q_len > k_len under bottom-right alignment: the first q_len - k_len rows see no key.
    q, k, v, cu_q, cu_k = make([10], [4], 2, 1, 3, seed=2)
    for fn in (oracle.attention, oracle.attention_chunked):
        o, l = fn(q, k, v, cu_q, cu_k, 2, 1, 1.0, True)
        assert np.all(o[:6] == 0.0) and np.all(np.isneginf(l[:6]))
        assert np.all(np.isfinite(l[6:]))
    # zero keys
    q, k, v, cu_q, cu_k = make([3], [0], 1, 1, 2, seed=2)
    o, l = oracle.attention(q, k, v, cu_q, cu_k, 1, 1, 1.0, False)
    assert np.all(o == 0.0) and np.all(np.isneginf(l))


def test_closed_forms():
    q, k, v, cu_q, cu_k = make([17, 1, 33], [17, 1, 33], 2, 1, 4, seed=11)
    o, l = oracle.attention(q, k, v, cu_q, cu_k, 2, 1, 0.7, True)
    # causal row 0 sees only key 0: O = V[0] and lse = scale * q0.k0
    for b in range(3):
        r = cu_q[b]
        for h in range(2):
            np.testing.assert_array_equal(o[r, h], v[cu_k[b], 0])
            assert l[r, h] == pytest.approx(0.7 * q[r, h] @ k[cu_k[b], 0], rel=1e-14)
    # q = 0: every visible key has score 0, so O is the mean of the visible V rows
    q0 = np.zeros_like(q)
    o, l = oracle.attention(q0, k, v, cu_q, cu_k, 2, 1, 0.7, True)
    for i in range(33):
        np.testing.assert_allclose(o[cu_q[2] + i, 1], v[cu_k[2]:cu_k[2] + i + 1, 0].mean(axis=0),
                                   rtol=1e-13, atol=1e-14)
        assert l[cu_q[2] + i, 1] == pytest.approx(math.log(i + 1), abs=1e-13)
    # one dominant score: O is that key's value row
    k2 = k.copy()
    q2 = np.zeros_like(q)
    q2[:, :, 0] = 1.0
    k2[:, :, 0] = 0.0
    k2[cu_k[2] + 5, 0, 0] = 2000.0
    o, _ = oracle.attention(q2, k2, v, cu_q, cu_k, 2, 1, 1.0, False)
    np.testing.assert_allclose(o[cu_q[2]:cu_q[3], 0], np.broadcast_to(v[cu_k[2] + 5, 0], (33, 4)),
                               atol=1e-300)


def test_two_key_closed_form():
    """softmax over two keys: weights e^a/(e^a+e^b), e^b/(e^a+e^b)."""
    q = np.array([[[1.0, 2.0]]])
    k = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    v = np.array([[[10.0, -1.0]], [[4.0, 3.0]]])
    o, l = oracle.attention(q, k, v, [0, 1], [0, 2], 1, 1, 0.5, False)
    a, b = 0.5, 1.0
    wa, wb = math.exp(a) / (math.exp(a) + math.exp(b)), math.exp(b) / (math.exp(a) + math.exp(b))
    np.testing.assert_allclose(o[0, 0], [10 * wa + 4 * wb, -1 * wa + 3 * wb], rtol=1e-15)
    assert l[0, 0] == pytest.approx(math.log(math.exp(a) + math.exp(b)), rel=1e-15)


def test_gqa_equals_repeated_mha():
    q, k, v, cu_q, cu_k = make([50, 20], [50, 20], 6, 2, 4, seed=4)
    o1, _ = oracle.attention(q, k, v, cu_q, cu_k, 6, 2, 0.3, True)
    o2, _ = oracle.attention(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), cu_q, cu_k, 6, 6,
                             0.3, True)
    np.testing.assert_array_equal(o1, o2)


def test_rows_subset_matches_full():
    q, k, v, cu_q, cu_k = make([100, 37], [100, 37], 2, 1, 4, seed=6)
    o, l = oracle.attention(q, k, v, cu_q, cu_k, 2, 1, 0.4, True)
    rows = [0, 5, 99, 100, 136]
    os_, ls = oracle.attention(q, k, v, cu_q, cu_k, 2, 1, 0.4, True, rows=rows)
    np.testing.assert_array_equal(os_[rows], o[rows])
    np.testing.assert_array_equal(ls[rows], l[rows])
    assert np.isnan(os_[1]).all()


def test_e4m3fn_table_spec_values():
    t = oracle.e4m3fn_table()
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and math.copysign(1, t[0x80]) == -1
    assert t[0x38] == 1.0            # exponent 7 = bias
    assert t[0x7E] == 448.0          # largest finite
    assert t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6      # smallest normal
    assert t[0x01] == 2.0 ** -9      # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9  # largest subnormal
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    fin = t[np.isfinite(t)]
    assert len(fin) == 254 and not np.isinf(t).any()
    pos = t[1:0x7F]
    assert np.all(np.diff(pos) > 0)  # codes 0x01..0x7E increase monotonically


def test_paged_decode_is_last_prefill_row():
    """A decode token at position ctx-1 equals the last row of the causal prefill
    of the same sequence (bottom-right alignment), whatever the page order."""
    rng = np.random.default_rng(8)
    hq, hkv, d, ps = 4, 2, 5, 16
    ctxs = [1, 16, 17, 100]
    seqs = [(rng.standard_normal((c, hq, d)), rng.standard_normal((c, hkv, d)),
             rng.standard_normal((c, hkv, d))) for c in ctxs]
    npages = sum((c + ps - 1) // ps for c in ctxs) + 3
    perm = rng.permutation(npages)
    kc = np.full((npages, ps, hkv, d), np.nan)
    vc = np.full((npages, ps, hkv, d), np.nan)
    table = np.zeros((len(ctxs), 7), dtype=np.int64)
    pos = 0
    for b, c in enumerate(ctxs):
        for j in range(c):
            if j % ps == 0:
                table[b, j // ps] = perm[pos]
                pos += 1
            kc[table[b, j // ps], j % ps] = seqs[b][1][j]
            vc[table[b, j // ps], j % ps] = seqs[b][2][j]
    qd = np.stack([s[0][-1] for s in seqs])
    o, l = oracle.paged_decode(qd, kc, vc, table, ctxs, hq, hkv, 0.45, ps)
    for b, c in enumerate(ctxs):
        qs, ks, vs = seqs[b]
        op, lp = brute_force(qs, ks, vs, [0, c], [0, c], hq, hkv, 0.45, True)
        np.testing.assert_allclose(o[b], op[-1], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(l[b], lp[-1], rtol=1e-12)


def test_flop_counts():
    f = oracle.attention_flops
    # dense: 4 * N^2 * D * H
    assert f([8192], [8192], 32, 128, False) == 4 * 8192 * 8192 * 128 * 32
    # causal, q_len == k_len: N(N+1)/2 pairs per head
    assert f([300], [300], 2, 64, True) == 4 * 64 * 2 * (300 * 301 // 2)
    lens = [4096, 2500, 1, 3969]
    assert f(lens, lens, 32, 128, True) == 4 * 128 * 32 * sum(n * (n + 1) // 2 for n in lens)
    # extend: the last row sees all keys
    assert f([2], [5], 1, 1, True) == 4 * (4 + 5)
    # q_len > k_len: leading rows see nothing
    assert f([5], [2], 1, 1, True) == 4 * (0 + 0 + 0 + 1 + 2)


# ---------------------------------------------------------------------------
# Sliding windows (local attention)
# ---------------------------------------------------------------------------
WINDOW_CASES = [
    # (seqlens_q, seqlens_k, causal, window)
    ([9], [9], True, (3, -1)),
    ([9], [9], False, (2, 4)),
    ([3, 9, 1], [3, 9, 1], True, (0, -1)),
    ([2, 5], [6, 11], True, (4, -1)),       # extend with a window
    ([6, 3], [4, 3], False, (1, 1)),        # q_len > k_len
    ([8], [8], False, (-1, 2)),             # right window only
]


@pytest.mark.parametrize("case", WINDOW_CASES)
def test_window_plain_matches_brute_force(case):
    sq, sk, causal, win = case
    q, k, v, cu_q, cu_k = make(sq, sk, 2, 1, 3, seed=sum(sk) + win[0] + 5 * win[1])
    o, l = oracle.attention(q, k, v, cu_q, cu_k, 2, 1, 0.41, causal, window=win)
    ob, lb = brute_force(q, k, v, cu_q, cu_k, 2, 1, 0.41, causal, window=win)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(l), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(l[fin], lb[fin], rtol=1e-12, atol=1e-13)


def test_window_zero_left_causal_closed_form():
    """With a left window of 0 under the causal mask each row sees exactly its
    own diagonal key: O_i = V[i + L_k - L_q] and lse_i = scale * q_i . k_diag."""
    sq, sk = [5, 4], [9, 4]
    q, k, v, cu_q, cu_k = make(sq, sk, 2, 2, 6, seed=3)
    o, l = oracle.attention(q, k, v, cu_q, cu_k, 2, 2, 0.5, True, window=(0, -1))
    for b in range(2):
        for i in range(sq[b]):
            j = cu_k[b] + i + sk[b] - sq[b]
            for h in range(2):
                np.testing.assert_allclose(o[cu_q[b] + i, h], v[j, h], rtol=0, atol=1e-15)
                np.testing.assert_allclose(l[cu_q[b] + i, h], 0.5 * q[cu_q[b] + i, h] @ k[j, h],
                                           rtol=1e-14)


def test_window_wide_equals_unwindowed():
    q, k, v, cu_q, cu_k = make([37, 5], [90, 70], 2, 1, 4, seed=9)
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, cu_q, cu_k, 2, 1, 0.3, causal)
        o2, l2 = oracle.attention(q, k, v, cu_q, cu_k, 2, 1, 0.3, causal, window=(500, 500))
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("win", [(100, -1), (700, -1), (64, 200)])
def test_window_chunked_equals_plain(win):
    """Windows that start and end inside chunks and blocks: the chunked
    evaluation skips nothing it should not (leading fully masked chunks stay
    empty) and equals the plain definition."""
    q, k, v, cu_q, cu_k = make([1300, 70], [1300, 1100], 2, 1, 8, seed=21)
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, cu_q, cu_k, 2, 1, 0.35, causal, window=win)
        o2, l2 = oracle.attention_chunked(q, k, v, cu_q, cu_k, 2, 1, 0.35, causal, window=win)
        np.testing.assert_allclose(o2, o1, rtol=1e-11, atol=1e-12)
        np.testing.assert_array_equal(np.isneginf(l1), np.isneginf(l2))


def test_window_flop_counts_match_mask():
    for sq, sk, causal, win in WINDOW_CASES + [([300], [300], True, (128, -1)),
                                              ([70], [1100], False, (64, 200))]:
        pairs = sum(int(oatt.visible(np.arange(a), a, b, causal, win).sum())
                    for a, b in zip(sq, sk))
        assert oracle.attention_flops(sq, sk, 3, 16, causal, window=win) == 4 * 16 * 3 * pairs


def test_window_decode_is_last_row():
    """A decode row with a left window equals the last row of the windowed
    causal prefill of the same sequence."""
    q, k, v, cu_q, cu_k = make([700], [700], 2, 1, 4, seed=5)
    o, l = oracle.attention(q, k, v, cu_q, cu_k, 2, 1, 0.5, True, window=(200, -1))
    page = 16
    pad = np.full((704 - 700, 1, 4), np.nan)  # dead slots of the last page
    kc = np.concatenate([k, pad]).reshape(-1, page, 1, 4)
    vc = np.concatenate([v, pad]).reshape(-1, page, 1, 4)
    table = np.arange(kc.shape[0])[None, :]
    od, ld = oracle.paged_decode(q[-1:], kc, vc, table, [700], 2, 1, 0.5, page, window_left=200)
    np.testing.assert_allclose(od[0], o[-1], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(ld[0], l[-1], rtol=1e-13)


def test_planted_window_off_by_one(monkeypatch):
    real = oatt.visible

    def strict(rows, lq, lk, causal, window=(-1, -1)):
        ok = real(rows, lq, lk, causal, window)
        if window[0] >= 0:  # drop the window's first key
            diag = np.asarray(rows)[:, None] + (lk - lq)
            ok = ok & (np.arange(lk)[None, :] > diag - window[0])
        return ok
    monkeypatch.setattr(oatt, "visible", strict)
    assert _fails(test_window_zero_left_causal_closed_form)
    assert _fails(lambda: test_window_plain_matches_brute_force(WINDOW_CASES[0]))


# ---------------------------------------------------------------------------
# Planted mistakes: each slip below is injected into the oracle (on the CPU) and
# at least one pin above must fail on it.
# ---------------------------------------------------------------------------
def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_top_left_causal_alignment(monkeypatch):
    def top_left(rows, lq, lk, causal, window=(-1, -1)):
        j = np.arange(lk)[None, :]
        ok = (j <= np.asarray(rows)[:, None]) if causal else (j < lk)
        return np.broadcast_to(ok, (len(rows), lk)).copy()
    monkeypatch.setattr(oatt, "visible", top_left)
    assert _fails(lambda: test_plain_matches_brute_force(SMALL_CASES[3]))


def test_planted_merge_without_rescale(monkeypatch):
    def bad_merge(total, part):
        M, L, A = total
        m, l, acc = part
        live = m > -np.inf
        return (np.where(live, np.maximum(M, m), M), L + np.where(live, l, 0),
                A + np.where(live[:, None], acc, 0))
    monkeypatch.setattr(oatt, "_merge", bad_merge)
    assert _fails(lambda: test_chunked_equals_plain(False, ([1300], [1300])))


def test_planted_block_update_without_alpha(monkeypatch):
    orig = oatt._block_update

    def no_alpha(state, s, vb):
        m, l, acc = state
        mblk = s.max(axis=1, initial=-np.inf)
        live = mblk > -np.inf
        m_new = np.where(live, np.maximum(m, mblk), m)
        p = np.where(live[:, None], np.exp(s - np.where(live, m_new, 0.0)[:, None]), 0.0)
        return m_new, l + p.sum(axis=1), acc + p @ vb
    monkeypatch.setattr(oatt, "_block_update", no_alpha)
    assert _fails(lambda: test_chunked_equals_plain(True, ([1300], [1300])))
    monkeypatch.setattr(oatt, "_block_update", orig)


def test_planted_e4m3_bias(monkeypatch):
    t = oracle.e4m3fn_table()
    bad = t * 2.0  # an exponent bias of 6 instead of 7
    monkeypatch.setattr(oracle, "e4m3fn_table", lambda: bad)
    assert _fails(test_e4m3fn_table_spec_values)


# ---------------------------------------------------------------------------
# E4M3FN dequantisation: decode(code) * per-tensor scale.  Every fp8 parity
# claim compares the GPU against the oracle on these values (ffpa-attn fp8
# D=192 page, "Verification": errors are taken against the dequantised inputs).
# ---------------------------------------------------------------------------
DEQ_SCALES = [1.0, 0.0123, 3.75, 2.0 ** -7]


@pytest.mark.parametrize("s", DEQ_SCALES)
def test_dequantize_e4m3_closed_forms(s):
    """Spec values of the OCP E4M3FN format times the scale, through the
    function the parity tests call (not the table)."""
    deq = oatt.dequantize_e4m3
    codes = np.array([0x38, 0x7E, 0xFE, 0x01, 0x08, 0x00, 0x80, 0xB8, 0x40, 0x30, 0x7F, 0xFF],
                     dtype=np.uint8)
    want = [1.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -6, 0.0, -0.0, -1.0, 2.0, 0.5]
    got = deq(codes, s)
    for c, w, g in zip(codes, want, got):
        assert g == w * s, f"code {c:#04x}: {g} != {w} * {s}"
    assert math.copysign(1.0, got[6]) == -1.0
    assert math.isnan(got[10]) and math.isnan(got[11])
    # shape is kept and every element is decoded independently
    grid = np.array([[0x38, 0x7E], [0x01, 0xB8]], dtype=np.uint8).reshape(2, 1, 2)
    np.testing.assert_array_equal(deq(grid, s), np.array([[[s, 448.0 * s]], [[2.0 ** -9 * s, -s]]]))


def test_dequantize_e4m3_matches_torch_decoder():
    """All 256 codes against torch's float8_e4m3fn conversion (an independent
    decoder of the same format), at several scales: decode exactly, then one
    fp64 multiply by the scale."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for s in DEQ_SCALES:
        got = oatt.dequantize_e4m3(codes, s)
        np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
        fin = ~np.isnan(ref)
        np.testing.assert_array_equal(got[fin], ref[fin] * np.float64(s))


def test_dequantize_inverts_per_tensor_quantisation():
    """Quantising x with the per-tensor amax/448 scale and dequantising gives x
    back within half an E4M3 step: relative 2^-4 for normal codes, absolute
    2^-10 * s below the smallest normal (2^-6 * s)."""
    import torch
    import synth
    x = torch.randn(4096, generator=torch.Generator().manual_seed(5)) * 3.0
    fq = synth.quantize_e4m3(x)
    back = oatt.dequantize_e4m3(fq.codes.numpy(), fq.scale)
    xs = x.double().numpy()
    s = fq.scale
    normal = np.abs(xs) >= 2.0 ** -6 * s
    assert normal.sum() > 3000 and (~normal).sum() > 0
    assert np.all(np.abs(back[normal] - xs[normal]) <= 2.0 ** -4 * np.abs(xs[normal]))
    assert np.all(np.abs(back[~normal] - xs[~normal]) <= 2.0 ** -10 * s * (1 + 1e-12))
    assert abs(np.abs(back).max() - np.abs(xs).max()) <= 2.0 ** -4 * np.abs(xs).max()


def _deq_pins():
    for s in DEQ_SCALES:
        test_dequantize_e4m3_closed_forms(s)
    test_dequantize_e4m3_matches_torch_decoder()
    test_dequantize_inverts_per_tensor_quantisation()


def test_planted_dequantize_divides_by_scale(monkeypatch):
    monkeypatch.setattr(oatt, "dequantize_e4m3",
                        lambda codes, scale: oatt._E4M3[np.asarray(codes, dtype=np.uint8)]
                        / np.float64(scale))
    assert _fails(_deq_pins)
    assert _fails(test_dequantize_inverts_per_tensor_quantisation)


def test_planted_dequantize_scales_code_before_decoding(monkeypatch):
    def scaled_first(codes, scale):
        c = np.asarray(codes, dtype=np.float64) * np.float64(scale)
        return oatt._E4M3[np.rint(c).astype(np.int64) % 256]
    monkeypatch.setattr(oatt, "dequantize_e4m3", scaled_first)
    assert _fails(lambda: test_dequantize_e4m3_closed_forms(0.0123))
    assert _fails(test_dequantize_e4m3_matches_torch_decoder)


def test_planted_dequantize_table_bias(monkeypatch):
    """A wrong exponent bias in the table dequantize_e4m3 actually reads."""
    monkeypatch.setattr(oatt, "_E4M3", oatt.e4m3fn_table() * 2.0)
    assert _fails(lambda: test_dequantize_e4m3_closed_forms(1.0))
    assert _fails(test_dequantize_e4m3_matches_torch_decoder)
    assert _fails(test_dequantize_inverts_per_tensor_quantisation)


def test_planted_dequantize_subnormal_slip(monkeypatch):
    """Subnormals decoded with the normal formula's implicit 1."""
    bad = oatt.e4m3fn_table().copy()
    for code in range(256):
        if (code >> 3) & 0xF == 0 and code & 0x7:
            sign = -1.0 if code & 0x80 else 1.0
            bad[code] = sign * (1.0 + (code & 7) / 8.0) * 2.0 ** -6
    monkeypatch.setattr(oatt, "_E4M3", bad)
    assert _fails(lambda: test_dequantize_e4m3_closed_forms(1.0))
    assert _fails(test_dequantize_e4m3_matches_torch_decoder)
