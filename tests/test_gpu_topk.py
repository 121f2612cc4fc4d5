"""GPU parity of sv_topk_candidates (through the C ABI) against the oracle:
ids and values exactly, in order, at the full vocabulary and on edge shapes
(ties everywhere, -inf entries, vocabularies that are not a multiple of 4 or
shorter than one slice, k = vocabulary), and on the workloads' logits."""
import numpy as np
import pytest
import torch

from helpers import say
from long_context_gqa_amd import binding as B
from long_context_gqa_amd import workloads as W
from oracle import topk as otk

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run(x, k):
    ids, vals = B.TopkCall(torch.tensor(x, device="cuda"), k).run()
    torch.cuda.synchronize()
    return ids.cpu().numpy(), vals.cpu().numpy()


def check(x, k, what=""):
    ids, vals = run(x, k)
    ri, rv = otk.topk(x, k)
    say(f"  {what}: rows {x.shape[0]} vocab {x.shape[1]} k {k}")
    np.testing.assert_array_equal(ids, ri)
    np.testing.assert_array_equal(vals, rv)


@pytest.mark.parametrize("rows,vocab,k", [
    (8, 248_320, 16), (64, 248_320, 16), (8, 248_320, 1), (8, 248_320, 5),
    (5, 1003, 16), (3, 100, 16), (4, 8192 * 3 + 5, 16), (2, 10, 10), (7, 8192, 16),
    # more than 64 rows: the narrower slices
    (100, 248_320, 16), (80, 8192 * 2 + 3, 7), (65, 1003, 16),
])
def test_random_rows(rows, vocab, k):
    rng = np.random.default_rng(rows * 1000 + vocab % 1000 + k)
    check((rng.standard_normal((rows, vocab)) * 3).astype(np.float32), k, "random")


@pytest.mark.parametrize("rows", [6, 70])
@pytest.mark.parametrize("vocab", [248_320, 1003])
def test_ties_everywhere_lowest_index_first(vocab, rows):
    rng = np.random.default_rng(vocab + rows)
    x = rng.integers(-3, 4, (rows, vocab)).astype(np.float32)
    check(x, 16, "integer ties")
    z = np.zeros((2, vocab), dtype=np.float32)
    ids, _ = run(z, 16)
    assert (ids == np.arange(16)).all()


def test_negative_infinity_and_few_finite_values():
    rng = np.random.default_rng(3)
    x = np.full((3, 50_000), -np.inf, dtype=np.float32)
    x[0, [7, 49_999, 20_000]] = [1.0, 2.0, 1.0]
    x[1, :] = rng.standard_normal(50_000).astype(np.float32)
    x[1, ::3] = -np.inf
    check(x, 16, "-inf")


@pytest.mark.parametrize("wl_id", [4, 3])
def test_workload_logits(wl_id):
    wl = W.WORKLOADS[wl_id]
    lg = W.make_accept_inputs(wl, device="cuda").logits
    ids, vals = B.TopkCall(lg, 16).run()
    torch.cuda.synchronize()
    ri, rv = otk.topk(lg.cpu().numpy(), 16)
    np.testing.assert_array_equal(ids.cpu().numpy(), ri)
    np.testing.assert_array_equal(vals.cpu().numpy(), rv)
