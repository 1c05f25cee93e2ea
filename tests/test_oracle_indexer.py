"""Pins of the oracle's block scores and exact top-k: special cases with a
closed form, brute force on tiny inputs, invariants, and the full
characterisation of the top-k answer (hypothesis)."""
import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import indexer as I


def _keys(L, seed=0):
    return np.random.default_rng(seed).standard_normal((L, 128))


def test_one_hot_query_is_columnwise_relu_max():
    """H_I = 1, w = 1, q_I = e_d: the score of block i is max(0, max_t k[t, d])
    over the block's visible tokens."""
    L, q = 700, 3
    k = _keys(L)
    for d in (0, 17, 127):
        qI = np.zeros((q, 1, 128))
        qI[:, 0, d] = 1.0
        S = I.index_scores(k, qI, np.ones((q, 1)), L)
        for j in range(q):
            pos = L - q + j
            for i in range(S.shape[1]):
                t1 = min(128 * i + 128, pos + 1)
                assert S[j, i] == max(0.0, k[128 * i:t1, d].max())


def test_scores_brute_force_tiny():
    rng = np.random.default_rng(1)
    L, q, H = 300, 2, 3
    k = rng.standard_normal((L, 128))
    qI = rng.standard_normal((q, H, 128))
    w = rng.random((q, H))
    S = I.index_scores(k, qI, w, L)
    for j in range(q):
        pos = L - q + j
        for i in range((L + 127) // 128):
            best = -np.inf
            for t in range(128 * i, min(128 * i + 128, L)):
                if t > pos:
                    continue
                tot = 0.0
                for h in range(H):
                    dot = sum(qI[j, h, d] * k[t, d] for d in range(128))
                    tot += w[j, h] * max(0.0, dot)
                best = max(best, tot)
            assert abs(S[j, i] - best) <= 1e-12 * max(1.0, abs(best))


def test_scores_positive_homogeneity_in_w_and_q():
    rng = np.random.default_rng(2)
    L, q = 513, 4
    k = rng.standard_normal((L, 128))
    qI = rng.standard_normal((q, 4, 128))
    w = rng.random((q, 4))
    S = I.index_scores(k, qI, w, L)
    np.testing.assert_allclose(I.index_scores(k, qI, 3.0 * w, L), 3.0 * S, rtol=1e-13)
    np.testing.assert_allclose(I.index_scores(k, 0.5 * qI, w, L), 0.5 * S, rtol=1e-13)
    # negating the query of every head turns ReLU(x) into ReLU(-x): all-negative
    # keys then score 0 against a positive query
    kneg = -np.abs(k)
    qpos = np.abs(qI)
    assert (I.index_scores(kneg, qpos, w, L)[np.isfinite(S)] == 0).all()


def test_scores_causal_and_candidate_count():
    rng = np.random.default_rng(3)
    L, q = 1000, 8
    k = rng.standard_normal((L, 128))
    qI = rng.standard_normal((q, 4, 128))
    w = rng.random((q, 4))
    S = I.index_scores(k, qI, w, L)
    nc = I.n_candidates(L, q)
    assert list(nc) == [(L - q + j) // 128 + 1 for j in range(q)]
    for j in range(q):
        assert np.isfinite(S[j, :nc[j]]).all() and np.isneginf(S[j, nc[j]:]).all()
    k2 = k.copy()
    k2[L - q + 3:] = 1e3                        # tokens after row 2's position
    S2 = I.index_scores(k2, qI, w, L)
    np.testing.assert_array_equal(S2[:3], S[:3])
    assert not np.array_equal(S2[3:], S[3:])


def test_zero_query_gives_lowest_ids():
    L, q = 2048, 1
    S = I.index_scores(_keys(L), np.zeros((q, 4, 128)), np.ones((q, 4)), L)
    assert (S == 0).all()
    assert list(I.topk_blocks(S[0], 16, 4)) == [0, 1, 2, 3]


def test_duplicated_pages_tie_to_lower_id():
    k = _keys(2048, 5)
    k[128 * 9:128 * 10] = k[128 * 2:128 * 3]    # block 9 duplicates block 2
    qI = np.zeros((1, 4, 128))
    qI[0, 0] = k[128 * 2 + 5] * 10              # block 2 (and 9) win by far
    S = I.index_scores(k, qI, np.ones((1, 4)), 2048)
    assert S[0, 2] == S[0, 9] == S[0].max()
    assert list(I.topk_blocks(S[0], 16, 1)) == [2]
    assert list(I.topk_blocks(S[0], 16, 2))[:2] == sorted([2, 9])


def test_fewer_candidates_than_k():
    s = np.array([3.0, 1.0, 2.0])
    assert list(I.topk_blocks(s, 3, 5)) == [0, 1, 2, -1, -1]


def test_kth_score_worked_values():
    s = np.array([1.0, 5.0, 3.0, 5.0, 2.0, -np.inf])
    assert I.kth_score(s, 5, 1) == 5.0
    assert I.kth_score(s, 5, 2) == 5.0          # a tie at the top counts twice
    assert I.kth_score(s, 5, 3) == 3.0
    assert I.kth_score(s, 5, 5) == 1.0
    assert I.kth_score(s, 5, 9) == 1.0          # fewer candidates than k: the smallest candidate
    assert I.kth_score(s, 2, 4) == 1.0          # only the first n_cand entries are candidates
    assert I.kth_score(s, 6, 6) == -np.inf


@settings(max_examples=300, deadline=None)
@given(st.lists(st.integers(-3, 3), min_size=1, max_size=40), st.integers(1, 50), st.integers(0, 40))
def test_kth_score_brute_force(vals, k, cut):
    """The k-th largest candidate score equals the score of the k-th member of
    the brute-force ordering by (score desc, id asc), and is the score of the
    lowest-ranked block top-k keeps."""
    s = np.array(vals, dtype=np.float64)
    n = max(1, min(len(vals), cut or len(vals)))
    ranked = sorted(range(n), key=lambda i: (-s[i], i))
    kk = min(k, n)
    assert I.kth_score(s, n, k) == s[ranked[kk - 1]]
    kept = [i for i in I.topk_blocks(s, n, k) if i >= 0]
    assert I.kth_score(s, n, k) == min(s[i] for i in kept)


@settings(max_examples=300, deadline=None)
@given(st.lists(st.integers(-3, 3), min_size=1, max_size=40), st.integers(1, 12))
def test_topk_characterisation(vals, k):
    """The answer is the unique set T with |T| = min(k, n), every member's
    score >= every non-member's, and among equal scores at the boundary the
    lower ids are members; listed ascending, padded with -1."""
    s = np.array(vals, dtype=np.float64)
    n = len(vals)
    out = I.topk_blocks(s, n, k)
    sel = [i for i in out if i >= 0]
    assert len(sel) == min(k, n) and (out[len(sel):] == -1).all()
    assert sel == sorted(sel)
    rest = [i for i in range(n) if i not in sel]
    for a in sel:
        for b in rest:
            assert s[a] > s[b] or (s[a] == s[b] and a < b)
