"""Pins of the top-k candidate oracle: brute-force selection, the library
sort for the values, the lowest-index tie rule, and the pages' claim that a
top-k of per-shard top-k lists gives the same candidates as the unsharded
row. A planted mistake (highest index first on ties) fails the tie pin."""
import numpy as np
import pytest

from oracle import topk as otk


def brute(row, k):
    # k rounds of: the largest remaining value, the lowest index among equals
    left = list(range(len(row)))
    out = []
    for _ in range(k):
        best = left[0]
        for i in left:
            if row[i] > row[best] or (row[i] == row[best] and i < best):
                best = i
        out.append(best)
        left.remove(best)
    return out


@pytest.mark.parametrize("seed", range(4))
def test_matches_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    row = rng.integers(-5, 6, 60).astype(np.float32)  # many ties
    for k in (1, 5, 16):
        idx, val = otk.topk_row(row, k)
        assert idx.tolist() == brute(row, k)
        np.testing.assert_array_equal(val, row[idx])


def test_values_are_the_library_sort():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, 5000)).astype(np.float32)
    idx, val = otk.topk(x, 16)
    np.testing.assert_array_equal(val, -np.sort(-x, axis=1)[:, :16])
    for r in range(6):
        assert set(idx[r].tolist()) == set(np.argpartition(-x[r], 16)[:16].tolist())


def test_sharded_top_k_gives_the_unsharded_candidates():
    rng = np.random.default_rng(10)
    for _ in range(20):
        row = rng.integers(-20, 20, 4000).astype(np.float32)
        cuts = np.sort(rng.choice(np.arange(1, 4000), 3, replace=False))
        bounds = [0, *cuts.tolist(), 4000]
        cand_i, cand_v = [], []
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            i, v = otk.topk_row(row[lo:hi], min(16, hi - lo))
            cand_i += (i + lo).tolist()
            cand_v += v.tolist()
        cand_i, cand_v = np.array(cand_i), np.array(cand_v)
        order = np.lexsort((cand_i, -cand_v.astype(np.float64)))[:16]
        gi, gv = otk.topk_row(row, 16)
        assert cand_i[order].tolist() == gi.tolist()


def test_planted_tie_rule_mistake_fails():
    row = np.array([3, 7, 7, 1, 7, 2], dtype=np.float32)
    idx, _ = otk.topk_row(row, 3)
    assert idx.tolist() == [1, 2, 4]

    def highest_index_first(r, k):
        order = np.lexsort((-np.arange(len(r)), -r.astype(np.float64)))
        return order[:k]
    assert highest_index_first(row, 3).tolist() != brute(row, 3)
