"""Pins of the block-preparation, KV-append and per-request-width oracle
functions against facts from outside each of them: a library prefix sum, the
attention oracle's own paged gather, pure-Python brute force on tiny inputs,
the uniform-width functions (written separately) when every width is equal,
and closed forms. ``test_ragged_pins_catch_planted_mistakes`` plants plausible
mistakes in copies of the functions and shows that the pins fail on them.
"""
import math

import numpy as np
import pytest

from oracle import accept as oacc
from oracle import attention as oatt
from oracle import block as oblk
from oracle import brute

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _table(rng, lens_total, P, num_pages):
    """A page table giving every request distinct random pages for its
    lens_total[b] positions (the reserved slots of the coming block included)."""
    need = [(n + P - 1) // P for n in lens_total]
    ids = rng.permutation(num_pages)[:sum(need)]
    t = np.full((len(need), max(need)), -1, dtype=np.int64)
    k = 0
    for b, n in enumerate(need):
        t[b, :n] = ids[k:k + n]
        k += n
    return t


def _case(seed=0, L=(5, 0, 9, 3), qn=(3, 1, 4, 2), P=4, Hkv=2, D=8):
    rng = np.random.default_rng(seed)
    L, qn = np.array(L), np.array(qn)
    num_pages = int(sum((L + qn + P - 1) // P)) + 3
    table = _table(rng, L + qn, P, num_pages)
    return rng, L, qn, P, Hkv, D, num_pages, table


def test_prepare_block_packing_is_the_prefix_sum_of_widths():
    rng, L, qn, P, Hkv, D, num_pages, table = _case()
    r = oblk.prepare_block(L, qn, table, P)
    np.testing.assert_array_equal(r["q_start"], np.concatenate([[0], np.cumsum(qn)]))
    np.testing.assert_array_equal(r["kv_lens_out"], L + qn)


def test_append_then_paged_gather_reads_the_block_back():
    # positions and cache slots, checked through the attention oracle's own
    # gather: after writing the block rows at their slots, reading request b's
    # cache in position order returns row q_start[b] + i at position L_b + i,
    # and nothing else in the pool changed
    rng, L, qn, P, Hkv, D, num_pages, table = _case(seed=1)
    r = oblk.prepare_block(L, qn, table, P)
    pool = rng.standard_normal((num_pages, Hkv, P, D))
    new = rng.standard_normal((int(qn.sum()), Hkv, D)) + 100.0
    pool2 = oblk.append_kv(pool, r["cache_slot"], new)
    for b in range(len(L)):
        for h in range(Hkv):
            rows = oatt.gather_kv(pool2, None, table[b], int(L[b] + qn[b]), h)
            for i in range(qn[b]):
                np.testing.assert_array_equal(rows[L[b] + i], new[r["q_start"][b] + i, h])
    changed = np.argwhere(pool2 != pool)
    assert len(changed) == new.size


def test_block_ids_and_ragged_accept_equal_the_uniform_accept():
    # equal widths: the packed block ids [t0, d1..] walked by the ragged accept
    # give what the uniform accept gives from the padded drafts
    rng = np.random.default_rng(2)
    B, q, V = 5, 6, 40
    L = rng.integers(0, 50, B)
    table = _table(rng, L + q, 16, 64)
    last = rng.integers(0, V, B)
    logits = rng.standard_normal((B * q, V))
    am = logits.argmax(axis=1).reshape(B, q)
    drafts = np.array([[am[b, j] if j < (b % q) else (am[b, j] + 1) % V for j in range(q - 1)] for b in range(B)])
    r = oblk.prepare_block(L, np.full(B, q), table, 16, last, drafts)
    a1, b1, _, n1 = oacc.greedy_accept_ragged(logits, r["block_ids"], np.full(B, q), r["q_start"], L + q)
    a2, b2, _, n2 = oacc.greedy_accept(logits, drafts, q, L + q)
    np.testing.assert_array_equal(a1, a2)
    np.testing.assert_array_equal(b1, b2)
    np.testing.assert_array_equal(n1, n2)
    np.testing.assert_array_equal(a1, [b % q for b in range(B)])


def test_ragged_accept_closed_forms():
    # width 1: nothing to accept, the bonus is the row's argmax (numpy's
    # first occurrence); a planted mismatch at draft k stops the walk at k
    rng = np.random.default_rng(3)
    V = 30
    qn = np.array([1, 4, 3, 1])
    qs = np.concatenate([[0], np.cumsum(qn)])
    logits = rng.standard_normal((int(qn.sum()), V))
    am = logits.argmax(axis=1)
    ids = np.zeros(int(qn.sum()), dtype=np.int64)
    ids[qs[1] + 1] = am[qs[1]]                 # request 1: d1 matches
    ids[qs[1] + 2] = (am[qs[1] + 1] + 1) % V   # d2 does not
    ids[qs[1] + 3] = am[qs[1] + 2]
    ids[qs[2] + 1] = am[qs[2]]                 # request 2: all drafts match
    ids[qs[2] + 2] = am[qs[2] + 1]
    acc, bonus, _, new = oacc.greedy_accept_ragged(logits, ids, qn, qs, np.array([10, 20, 30, 40]))
    np.testing.assert_array_equal(acc, [0, 1, 2, 0])
    np.testing.assert_array_equal(bonus, [am[0], am[qs[1] + 1], am[qs[2] + 2], am[qs[3]]])
    np.testing.assert_array_equal(new, [10, 20 - 4 + 2, 30 - 3 + 3, 40])


def _ragged_inputs(seed, L, qn, Hq=4, Hkv=2, D=8, P=4):
    rng = np.random.default_rng(seed)
    L, qn = np.array(L), np.array(qn)
    kv = L + qn
    num_pages = int(sum((kv + P - 1) // P)) + 2
    table = _table(rng, kv, P, num_pages)
    kp = rng.standard_normal((num_pages, Hkv, P, D))
    vp = rng.standard_normal((num_pages, Hkv, P, D))
    qs = np.concatenate([[0], np.cumsum(qn)])
    q = rng.standard_normal((int(qs[-1]), Hq, D))
    return q, kp, vp, table, kv, qn, qs, 1.0 / math.sqrt(D)


def test_ragged_attention_matches_brute_force_rows():
    q, kp, vp, table, kv, qn, qs, sm = _ragged_inputs(4, [3, 0, 7], [2, 3, 1])
    out, lse = oatt.verify_attention_ragged(q, kp, vp, table, kv, qn, qs, sm)
    P, G = kp.shape[2], q.shape[1] // kp.shape[1]
    for b in range(len(kv)):
        for i in range(qn[b]):
            n = kv[b] - qn[b] + i + 1
            for h in range(q.shape[1]):
                g = h // G
                keys = [kp[table[b, t // P], g, t % P].tolist() for t in range(n)]
                vals = [vp[table[b, t // P], g, t % P].tolist() for t in range(n)]
                bo, bl = brute.attention_row(q[qs[b] + i, h].tolist(), keys, vals, sm)
                np.testing.assert_allclose(out[qs[b] + i, h], bo, rtol=0, atol=1e-13)
                assert abs(lse[qs[b] + i, h] - bl) < 1e-13


def test_ragged_attention_equal_widths_equal_the_uniform_oracle():
    q, kp, vp, table, kv, qn, qs, sm = _ragged_inputs(5, [4, 9, 2], [3, 3, 3])
    o1, l1 = oatt.verify_attention_ragged(q, kp, vp, table, kv, qn, qs, sm)
    o2, l2 = oatt.verify_attention(q, kp, vp, table, kv, 3, sm)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


def test_ragged_attention_each_request_equals_its_own_uniform_call():
    q, kp, vp, table, kv, qn, qs, sm = _ragged_inputs(6, [6, 1, 11, 0], [1, 4, 2, 3])
    out, lse = oatt.verify_attention_ragged(q, kp, vp, table, kv, qn, qs, sm)
    for b in range(len(kv)):
        o, l = oatt.verify_attention(q[qs[b]:qs[b + 1]], kp, vp, table[b:b + 1], kv[b:b + 1], int(qn[b]), sm)
        np.testing.assert_allclose(out[qs[b]:qs[b + 1]], o, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[qs[b]:qs[b + 1]], l, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# planted mistakes: each must fail at least one of the pins above

def _mutant_attention_max_width(q, kp, vp, table, kv, qn, qs, sm, k_scales=None, v_scales=None, groups=None):
    # causal offset taken from the largest width instead of the request's own
    qmax = int(qn.max())
    Hq, Hkv = q.shape[1], kp.shape[1]
    G = Hq // Hkv
    out = np.zeros(q.shape)
    lse = np.zeros(q.shape[:2])
    for b in range(len(kv)):
        for g in range(Hkv):
            K = oatt.gather_kv(kp, None, table[b], int(kv[b]), g)
            V = oatt.gather_kv(vp, None, table[b], int(kv[b]), g)
            for i in range(qn[b]):
                n = max(1, int(kv[b]) - qmax + i + 1)
                for h in range(g * G, g * G + G):
                    s_ = sm * (K[:n] @ q[qs[b] + i, h])
                    w = np.exp(s_ - s_.max())
                    out[qs[b] + i, h] = (w @ V[:n]) / w.sum()
                    lse[qs[b] + i, h] = s_.max() + np.log(w.sum())
    return out, lse


def _mutant_accept_same_row(logits, ids, qn, qs, kv=None):
    # the draft compared with its own row instead of the previous one
    am = np.argmax(np.asarray(logits), axis=-1)
    B = len(qn)
    acc = np.zeros(B, dtype=np.int64)
    for b in range(B):
        a = 0
        while a < qn[b] - 1 and ids[qs[b] + a] == am[qs[b] + a]:
            a += 1
        acc[b] = a
    return acc, am[qs[:-1] + acc], am, None


def test_ragged_pins_catch_planted_mistakes(monkeypatch):
    with monkeypatch.context() as m:
        m.setattr(oatt, "verify_attention_ragged", _mutant_attention_max_width)
        with pytest.raises(AssertionError):
            test_ragged_attention_matches_brute_force_rows()
    with monkeypatch.context() as m:
        m.setattr(oacc, "greedy_accept_ragged", _mutant_accept_same_row)
        with pytest.raises(AssertionError):
            test_ragged_accept_closed_forms()
