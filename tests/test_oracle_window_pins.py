"""Pins of the sink + sliding-window verify oracle: a window that covers the
whole context (and window 0) is full attention — the page's own check — a
one-position window returns the row's own V exactly, brute force on tiny
inputs, and equality with full attention over a cache rebuilt from only the
visible keys. A planted off-by-one window fails the one-position pin."""
import math

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import brute


def case(seed, lens, q_len, P=4, Hq=4, Hkv=2, D=8):
    rng = np.random.default_rng(seed)
    npg = [(n + P - 1) // P for n in lens]
    num_pages = sum(npg) + 2
    perm = rng.permutation(num_pages)
    table = np.full((len(lens), max(npg)), -1, dtype=np.int64)
    k = 0
    for b, n in enumerate(npg):
        table[b, :n] = perm[k:k + n]
        k += n
    kp = rng.standard_normal((num_pages, Hkv, P, D))
    vp = rng.standard_normal((num_pages, Hkv, P, D))
    q = rng.standard_normal((len(lens) * q_len, Hq, D))
    return q, kp, vp, table, np.array(lens), 1 / math.sqrt(D)


def test_covering_window_and_window_zero_are_full_attention():
    q, kp, vp, t, kv, sm = case(0, [37, 20, 64], 4)
    ref, rl = oatt.verify_attention(q, kp, vp, t, kv, 4, sm)
    for W, S in ((0, 0), (0, 5), (64, 0), (1000, 3)):
        o, l = oatt.verify_attention_window(q, kp, vp, t, kv, 4, sm, W, S)
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, rl, rtol=0, atol=1e-13)


def test_one_position_window_returns_the_rows_own_value():
    q, kp, vp, t, kv, sm = case(1, [30, 9], 3)
    o, l = oatt.verify_attention_window(q, kp, vp, t, kv, 3, sm, 1, 0)
    G = 2
    for b in range(2):
        for i in range(3):
            pos = kv[b] - 3 + i
            for h in range(4):
                g = h // G
                vrow = vp[t[b, pos // 4], g, pos % 4]
                krow = kp[t[b, pos // 4], g, pos % 4]
                np.testing.assert_array_equal(o[b * 3 + i, h], vrow)
                assert abs(l[b * 3 + i, h] - sm * float(q[b * 3 + i, h] @ krow)) < 1e-12


@pytest.mark.parametrize("W,S", [(3, 0), (5, 2), (2, 7), (8, 1)])
def test_brute_force_rows(W, S):
    q, kp, vp, t, kv, sm = case(2, [19, 12], 3)
    o, l = oatt.verify_attention_window(q, kp, vp, t, kv, 3, sm, W, S)
    for b in range(2):
        for i in range(3):
            pos = kv[b] - 3 + i
            vis = [u for u in range(pos + 1) if u < S or u > pos - W]
            for h in range(4):
                g = h // 2
                keys = [kp[t[b, u // 4], g, u % 4].tolist() for u in vis]
                vals = [vp[t[b, u // 4], g, u % 4].tolist() for u in vis]
                bo, bl = brute.attention_row(q[b * 3 + i, h].tolist(), keys, vals, sm)
                np.testing.assert_allclose(o[b * 3 + i, h], bo, rtol=0, atol=1e-13)
                assert abs(l[b * 3 + i, h] - bl) < 1e-13


def test_equals_full_attention_over_the_visible_keys():
    # a one-row block: rebuild a cache holding only the visible keys, in
    # order, and run the full-attention oracle on it
    q, kp, vp, t, kv, sm = case(3, [50], 1, P=1)
    for W, S in ((6, 3), (11, 0), (4, 10)):
        o, l = oatt.verify_attention_window(q, kp, vp, t, kv, 1, sm, W, S)
        vis = oatt.visible_keys(int(kv[0]) - 1, W, S)
        t2 = t[:, vis]
        f, fl = oatt.verify_attention(q, kp, vp, t2, np.array([len(vis)]), 1, sm)
        np.testing.assert_allclose(o, f, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, fl, rtol=0, atol=1e-13)


def test_planted_off_by_one_window_fails():
    real = oatt.visible_keys
    try:
        oatt.visible_keys = lambda pos, w, s: np.arange(pos + 1) if w == 0 else \
            np.arange(pos + 1)[(np.arange(pos + 1) < s) | (np.arange(pos + 1) >= pos - w)]
        with pytest.raises(AssertionError):
            test_one_position_window_returns_the_rows_own_value()
    finally:
        oatt.visible_keys = real
