"""Pins of the rejection-sampling acceptance oracle against facts outside it:
a library softmax, brute-force inverse CDF, and the theorem that makes
speculative sampling exact — the first committed token is distributed as the
target's p_0 whatever the draft's distribution — checked by integrating the
oracle's decisions over fine uniform grids. Planted mistakes (acceptance ratio
inverted, residual sign flipped) fail it."""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import sampling as osm


def test_target_probs_is_the_library_softmax():
    rng = np.random.default_rng(0)
    for T in (0.3, 1.0, 2.5):
        l = rng.standard_normal(1000) * 4
        np.testing.assert_allclose(osm.target_probs(l, T), softmax(l / T), rtol=1e-12, atol=0)


def test_inverse_cdf_brute_force_and_frequencies():
    rng = np.random.default_rng(1)
    w = rng.random(7) * (rng.random(7) > 0.3)
    w[3] = 0.25
    tot = w.sum()
    for u in rng.random(200):
        run, want = 0.0, None
        for v in range(len(w)):
            run += w[v]
            if run > u * tot:
                want = v
                break
        assert osm.inverse_cdf(w, u) == want
    # on a grid of N midpoints each index is drawn N * w_v / sum(w) times (+-1)
    N = 4000
    hist = np.bincount([osm.inverse_cdf(w, (k + 0.5) / N) for k in range(N)], minlength=len(w))
    assert np.all(np.abs(hist - N * w / tot) <= 1.0)
    assert np.all(hist[w == 0] == 0)


def _first_token_law(accept_fn, logits_row, qdist, T, N=1000):
    """P(first committed token = v) for one draft position: d ~ q; kept with
    the accept function's rule, else replaced by the final draw. Integrated
    over grids of N midpoints for both uniforms."""
    V = len(qdist)
    logits = np.stack([logits_row, logits_row])  # row 1 only matters if kept
    law = np.zeros(V)
    grid = (np.arange(N) + 0.5) / N
    for d in range(V):
        if qdist[d] == 0:
            continue
        dq = np.stack([qdist, qdist])[None]
        kept = 0
        for u in grid:
            a, _, _ = accept_fn(logits, np.array([[d]]), dq, 2, T, np.array([[u]]), np.array([0.5]))
            kept += a[0]
        kept /= N
        law[d] += qdist[d] * kept
        if kept < 1:
            # rejected: the first committed token is the final draw (u_accept = 1 - 1e-12 rejects
            # whenever rejection is possible)
            hist = np.zeros(V)
            for u in grid:
                a, t, _ = accept_fn(logits, np.array([[d]]), dq, 2, T, np.array([[1 - 1e-12]]), np.array([u]))
                assert a[0] == 0
                hist[t[0]] += 1
            law += qdist[d] * (1 - kept) * hist / N
    return law


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_first_committed_token_has_the_target_law(seed):
    rng = np.random.default_rng(seed)
    V, T = 5, 0.8
    l = rng.standard_normal(V) * 2
    q = rng.dirichlet(np.ones(V))
    law = _first_token_law(osm.rejection_accept, l, q, T)
    np.testing.assert_allclose(law, softmax(l / T), atol=3e-3)


def test_planted_mistakes_break_the_target_law():
    rng = np.random.default_rng(7)
    V, T = 5, 0.8
    l = rng.standard_normal(V) * 2
    q = rng.dirichlet(np.ones(V))
    p = softmax(l / T)

    def inverted_ratio(logits, ids, dq, q_len, T_, ua, uf, kv=None):
        # accept with probability min(1, q/p) instead of min(1, p/q)
        d = ids[0, 0]
        pp = osm.target_probs(logits[0], T_)
        if ua[0, 0] * pp[d] < dq[0, 0, d]:
            return np.array([1]), np.array([osm.inverse_cdf(osm.target_probs(logits[1], T_), uf[0])]), None
        r = np.maximum(pp - dq[0, 0], 0)
        return np.array([0]), np.array([osm.inverse_cdf(r if r.sum() > 0 else pp, uf[0])]), None

    def flipped_residual(logits, ids, dq, q_len, T_, ua, uf, kv=None):
        d = ids[0, 0]
        pp = osm.target_probs(logits[0], T_)
        if ua[0, 0] * dq[0, 0, d] < pp[d]:
            return np.array([1]), np.array([osm.inverse_cdf(osm.target_probs(logits[1], T_), uf[0])]), None
        r = np.maximum(dq[0, 0] - pp, 0)
        return np.array([0]), np.array([osm.inverse_cdf(r if r.sum() > 0 else pp, uf[0])]), None

    for bad in (inverted_ratio, flipped_residual):
        law = _first_token_law(bad, l, q, T, N=400)
        assert np.abs(law - p).max() > 0.02, bad.__name__


def test_draft_equal_to_target_accepts_everything():
    rng = np.random.default_rng(3)
    B, q_len, V, T = 3, 6, 50, 1.3
    logits = rng.standard_normal((B * q_len, V))
    dq = np.stack([[softmax(logits[b * q_len + j] / T) for j in range(q_len - 1)] for b in range(B)])
    ids = rng.integers(0, V, (B, q_len - 1))
    ua = rng.random((B, q_len - 1)) * 0.999
    uf = rng.random(B)
    acc, tok, new = osm.rejection_accept(logits, ids, dq, q_len, T, ua, uf, np.array([100, 200, 300]))
    np.testing.assert_array_equal(acc, q_len - 1)
    for b in range(B):
        assert tok[b] == osm.inverse_cdf(softmax(logits[b * q_len + q_len - 1] / T), uf[b])
    np.testing.assert_array_equal(new, np.array([100, 200, 300]) - q_len + 1 + acc)


def test_impossible_draft_is_rejected_and_never_redrawn():
    # p(d) = 0 at row 1: d_2 is rejected for every u, and the redraw never
    # returns d_2 (the residual is zero there)
    V, T, q_len = 6, 1.0, 3
    logits = np.zeros((q_len, V))
    logits[1, 4] = -1e4
    dq = np.full((1, q_len - 1, V), 1.0 / V)
    ids = np.array([[2, 4]])
    for u in (0.0, 0.3, 0.99):
        for uf in (0.01, 0.5, 0.99):
            acc, tok, _ = osm.rejection_accept(logits, ids, dq, q_len, T, np.array([[u, u]]), np.array([uf]))
            assert acc[0] == 1 and tok[0] != 4


def test_no_drafts_is_a_plain_draw_from_row_zero():
    rng = np.random.default_rng(5)
    B, V, T = 4, 30, 0.7
    logits = rng.standard_normal((B, V))
    uf = rng.random(B)
    acc, tok, new = osm.rejection_accept(logits, np.zeros((B, 0), int), np.zeros((B, 0, V)), 1, T,
                                         np.zeros((B, 0)), uf, np.full(B, 9))
    np.testing.assert_array_equal(acc, 0)
    np.testing.assert_array_equal(new, 9)  # kv_len - 1 + 1 + 0: the drawn token is not cached yet
    for b in range(B):
        assert tok[b] == osm.inverse_cdf(softmax(logits[b] / T), uf[b])
