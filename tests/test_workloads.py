"""The seeded input generator: determinism, layouts, planted accept lengths
(checked by the oracle, not by the generator), poison placement."""
import hashlib

import numpy as np
import pytest
import torch

from long_context_gqa_amd import workloads as W
from oracle import accept as oacc


def small(wl_id, **kw):
    wl = W.WORKLOADS[wl_id]
    base = dict(batch=min(wl.batch, 3), prefix=("fixed", 100))
    if wl.prefix[0] == "uniform":
        base["prefix"] = ("uniform", 60, 200)
    base.update(kw)
    return wl.with_(**base)


def _digest(*ts):
    h = hashlib.sha256()
    for t in ts:
        if t is not None:
            h.update(t.contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("wl_id", [1, 2, 3, 4, 5])
def test_generator_is_deterministic(wl_id):
    wl = small(wl_id)
    a = W.make_verify_inputs(wl)
    b = W.make_verify_inputs(wl)
    assert _digest(a.q, a.k_pages, a.v_pages, a.k_scales, a.v_scales, a.page_table) == \
        _digest(b.q, b.k_pages, b.v_pages, b.k_scales, b.v_scales, b.page_table)
    c = W.make_verify_inputs(wl.with_(seed=wl.seed + 1))
    assert _digest(a.k_pages) != _digest(c.k_pages)


@pytest.mark.parametrize("wl_id", [1, 4])
def test_page_tables_are_permutations_and_poison_is_outside(wl_id):
    wl = small(wl_id)
    x = W.make_verify_inputs(wl)
    P = wl.page_size
    used = []
    for b, n in enumerate(x.kv_lens.tolist()):
        npg = (n + P - 1) // P
        row = x.page_table[b]
        assert (row[:npg] >= 0).all() and (row[:npg] < x.num_pages).all()
        assert (row[npg:] == -1).all()
        used += row[:npg].tolist()
        # valid slots are finite, the tail of the last page is NaN
        for t in range(n):
            assert torch.isfinite(x.k_pages[row[t // P], :, t % P].float()).all()
        if n % P:
            assert torch.isnan(x.v_pages[row[npg - 1], :, n % P:].float()).all()
    assert len(set(used)) == len(used)
    spare = sorted(set(range(x.num_pages)) - set(used))
    assert spare and torch.isnan(x.k_pages[spare].float()).all()


def test_value_scales_of_the_variants():
    wl = W.WORKLOADS[2].with_(batch=1, prefix=("fixed", 4096))
    lit = W.make_verify_inputs(wl, "literal", poison=False)
    uni = W.make_verify_inputs(wl, "unit", poison=False)
    assert abs(lit.k_pages.float().std().item() - 1 / 16) < 2e-3
    assert abs(uni.k_pages.float().std().item() - 1.0) < 2e-2
    assert abs(lit.q.float().std().item() - 1 / 16) < 2e-3


def test_fp8_codes_and_scales():
    wl = small(5)
    x = W.make_verify_inputs(wl, poison=False)
    assert x.k_pages.dtype == torch.uint8 and x.k_scales.dtype == torch.float16
    assert x.k_scales.shape == (x.num_pages, 4, wl.page_size, 4)
    codes = x.k_pages.flatten()
    assert not ((codes & 0x7F) == 0x7F).any()  # no NaN codes in data
    # each 64-channel block uses the top code magnitude (amax maps to ~448)
    mags = (x.k_pages & 0x7F).view(x.num_pages, 4, wl.page_size, 4, 64).amax(-1)
    assert (mags >= 0x7D).float().mean() > 0.99


def test_bias_keys_include_block_and_page_boundary():
    wl = small(3)
    x = W.make_verify_inputs(wl)
    assert x.bias_positions
    for b, g, pos in x.bias_positions:
        n = int(x.kv_lens[b])
        L = n - wl.q_len
        assert any(L <= t < n for t in pos)
        assert any(t % wl.page_size == 0 for t in pos)


@pytest.mark.parametrize("wl_id", [1, 2, 4])
def test_planted_accept_lengths_are_what_the_oracle_returns(wl_id):
    wl = W.WORKLOADS[wl_id].with_(vocab=5000)
    a = W.make_accept_inputs(wl)
    acc, bonus, am, _ = oacc.greedy_accept(a.logits.numpy(), a.draft_ids.numpy(), wl.q_len)
    np.testing.assert_array_equal(acc, a.planted_accept.numpy())
    for b in range(wl.batch):
        assert bonus[b] == a.planted_targets[b, acc[b]]
    if wl.accept_dist == "uniform":
        assert acc.max() <= wl.q_len - 1
    else:
        assert acc.max() <= 15


def test_full_size_byte_counts():
    # config-level algorithmic bytes used by the benchmark
    wl = W.WORKLOADS[3]
    kv = [L + wl.q_len for L in W.prefix_lengths(wl)]
    b = W.verify_algorithmic_bytes(kv, wl.q_len, 24, 4, 256, wl.page_size, "fp16")
    assert b == 524296 * 4 * 1024 + 2 * 8 * 24 * 256 * 2 + 32769 * 4 + 4
    wl5 = W.WORKLOADS[5]
    kv5 = [L + wl5.q_len for L in W.prefix_lengths(wl5)]
    b5 = W.verify_algorithmic_bytes(kv5, 8, 24, 4, 256, 16, "fp8_e4m3")
    assert b5 == 4 * 262152 * 4 * 528 + 2 * 32 * 24 * 256 * 2 + 4 * 16385 * 4 + 16
