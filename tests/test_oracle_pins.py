"""Pins of the CPU oracle against facts that do not come from the oracle itself:
values printed on the pages, closed forms, a library routine, brute force on
tiny inputs and invariants of the definition. Each check is chosen so that a
plausible mistake in the oracle (causal off-by-one, wrong GQA grouping, a
transposed operand, a dropped scale, a wrong tie rule) fails at least one of
them; ``test_pins_catch_planted_mistakes`` plants such mistakes in copies of
the oracle and shows that they do.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import accept as oacc
from oracle import attention as oatt
from oracle import brute
from oracle import fp8 as ofp8

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------------------
# helpers building small paged caches by hand (no generator involved)

def paged(kv_rows, P, perm_seed=None, spare=1):
    """Lay per-request, per-KV-head rows [B][g][n][D] into a paged pool.
    Returns (pages [num_pages, Hkv, P, D], page_table [B, maxp])."""
    B = len(kv_rows)
    Hkv = len(kv_rows[0])
    D = len(kv_rows[0][0][0])
    npg = [(len(kv_rows[b][0]) + P - 1) // P for b in range(B)]
    total = sum(npg) + spare
    ids = np.arange(total)
    if perm_seed is not None:
        ids = np.random.default_rng(perm_seed).permutation(total)
    pages = np.full((total, Hkv, P, D), np.nan, dtype=np.float64)
    table = np.full((B, max(npg)), -1, dtype=np.int64)
    k = 0
    for b in range(B):
        for p in range(npg[b]):
            table[b, p] = ids[k]
            k += 1
        for g in range(Hkv):
            for t, row in enumerate(kv_rows[b][g]):
                pages[table[b, t // P], g, t % P] = row
    return pages, table


def rand_case(rng, B, q_len, Hq, Hkv, D, P, lens, scale=1.0):
    q = rng.standard_normal((B * q_len, Hq, D)) * scale
    K = [[rng.standard_normal((lens[b], D)) * scale for _ in range(Hkv)] for b in range(B)]
    V = [[rng.standard_normal((lens[b], D)) for _ in range(Hkv)] for b in range(B)]
    kp, table = paged(K, P, perm_seed=int(rng.integers(1 << 30)))
    # the same physical placement for V: rebuild with the same table
    vp = np.full_like(kp, np.nan)
    for b in range(B):
        for g in range(Hkv):
            for t in range(lens[b]):
                vp[table[b, t // P], g, t % P] = V[b][g][t]
    return q, kp, vp, table, np.array(lens)


# ---------------------------------------------------------------------------
# attention: brute force on tiny inputs

@pytest.mark.parametrize("B,q_len,Hq,Hkv,D,P,lens", [
    (1, 1, 2, 1, 8, 4, [5]),
    (2, 3, 4, 2, 8, 4, [7, 12]),
    (1, 4, 6, 2, 16, 16, [21]),
    (3, 2, 2, 2, 4, 4, [2, 9, 16]),
    (1, 40, 2, 1, 4, 4, [45]),       # an extend chunk longer than the verify blocks
    (2, 24, 2, 2, 4, 4, [24, 30]),   # a prefill with no prefix (L = 0) and one with L = 6
])
def test_attention_matches_fsum_brute_force(B, q_len, Hq, Hkv, D, P, lens):
    rng = np.random.default_rng(7)
    q, kp, vp, table, kv = rand_case(rng, B, q_len, Hq, Hkv, D, P, lens)
    sm = 1.0 / math.sqrt(D)
    out, lse = oatt.verify_attention(q, kp, vp, table, kv, q_len, sm)
    bo, bl = brute.verify_attention(q.tolist(), kp.tolist(), vp.tolist(), table.tolist(),
                                    kv.tolist(), q_len, sm)
    np.testing.assert_allclose(out, np.array(bo), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, np.array(bl), rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# attention: closed forms

def _probe_case(L, q_len, P, Hq, Hkv, D, planted, seed=3):
    """Unit-size position probe: query of head h = 8*u_h, key at position
    planted[(b, g)] = 8*u_h; every other key 0. With D = 256 and scale 1/16
    the planted logit is 8*8*256/16 = 1024 and every other logit 0, so the
    softmax is exactly one-hot (exp(-1024) underflows to 0 in float64)."""
    rng = np.random.default_rng(seed)
    n = L + q_len
    G = Hq // Hkv
    u = rng.choice([-1.0, 1.0], size=(Hkv, D))
    q = np.zeros((q_len, Hq, D))
    for h in range(Hq):
        q[:, h] = 8.0 * u[h // G]
    K = [[np.zeros((n, D)) for _ in range(Hkv)]]
    for g in range(Hkv):
        t = planted[g]
        if t is not None and t < n:
            K[0][g][t] = 8.0 * u[g]
    V = [[rng.integers(-64, 65, size=(n, D)) / 64.0 for _ in range(Hkv)]]
    kp, table = paged(K, P, perm_seed=seed)
    vp = np.full_like(kp, np.nan)
    for g in range(Hkv):
        for t in range(n):
            vp[table[0, t // P], g, t % P] = V[0][g][t]
    return q, kp, vp, table, np.array([n]), V[0]


@pytest.mark.parametrize("P", [4, 16])
def test_position_probe_one_hot_and_causal_edge(P):
    L, q_len, Hq, Hkv, D = 3 * P - 1, 4, 6, 2, 256
    for i in range(q_len):
        for delta, visible in ((0, True), (1, False)):
            t_star = L + i + delta  # L+i is row i's last visible key, L+i+1 the first hidden
            q, kp, vp, table, kv, V = _probe_case(L, q_len, P, Hq, Hkv, D, [t_star, 0])
            out, _ = oatt.verify_attention(q, kp, vp, table, kv, q_len, 1.0 / 16)
            row = out[i]
            # KV head 0: planted at t_star; heads 0..2 use it
            if visible:
                for h in range(3):
                    assert np.array_equal(row[h], V[0][t_star])
            else:
                mean = V[0][:L + i + 1].mean(axis=0)
                for h in range(3):
                    np.testing.assert_allclose(row[h], mean, atol=1e-14)
            # KV head 1 planted at position 0 (always visible): heads 3..5
            for h in range(3, 6):
                assert np.array_equal(row[h], V[1][0])


def test_position_probe_across_page_boundaries():
    P, L, q_len, Hq, Hkv, D = 16, 100, 2, 4, 2, 256
    for t_star in (0, 15, 16, 17, 31, 32, 63, 64, 99, 100):
        q, kp, vp, table, kv, V = _probe_case(L, q_len, P, Hq, Hkv, D, [t_star, t_star // 2])
        out, _ = oatt.verify_attention(q, kp, vp, table, kv, q_len, 1.0 / 16)
        for i in range(q_len):
            assert np.array_equal(out[i, 0], V[0][t_star])
            assert np.array_equal(out[i, 2], V[1][t_star // 2])


def test_zero_query_gives_exact_mean_of_visible_values():
    rng = np.random.default_rng(11)
    P, q_len, Hq, Hkv, D = 4, 3, 4, 2, 8
    lens = [9, 14]
    V = [[rng.integers(-100, 101, size=(n, D)) for _ in range(Hkv)] for n in lens]
    K = [[rng.standard_normal((n, D)) for _ in range(Hkv)] for n in lens]
    kp, table = paged(K, P, perm_seed=5)
    vp = np.full_like(kp, np.nan)
    for b in range(2):
        for g in range(Hkv):
            for t in range(lens[b]):
                vp[table[b, t // P], g, t % P] = V[b][g][t] / 64.0
    q = np.zeros((2 * q_len, Hq, D))
    out, lse = oatt.verify_attention(q, kp, vp, table, np.array(lens), q_len, 0.5)
    for b in range(2):
        L = lens[b] - q_len
        for i in range(q_len):
            n = L + i + 1
            for h in range(Hq):
                g = h // 2
                exact = [Fraction(int(sum(V[b][g][t][c] for t in range(n))), 64 * n) for c in range(D)]
                np.testing.assert_allclose(out[b * q_len + i, h], [float(x) for x in exact], rtol=0, atol=1e-15)
                assert abs(lse[b * q_len + i, h] - math.log(n)) < 1e-14  # all logits 0 -> lse = ln n


# ---------------------------------------------------------------------------
# attention: invariants of the definition

def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(2)
    B, q_len, Hq, Hkv, D, P = 2, 3, 6, 2, 16, 4
    q, kp, vp, table, kv = rand_case(rng, B, q_len, Hq, Hkv, D, P, [10, 13])
    out, lse = oatt.verify_attention(q, kp, vp, table, kv, q_len, 0.25)
    G = Hq // Hkv
    kp6 = np.repeat(kp, G, axis=1)  # KV head h//G copied to position h
    vp6 = np.repeat(vp, G, axis=1)
    out6, lse6 = oatt.verify_attention(q, kp6, vp6, table, kv, q_len, 0.25)
    # equal up to the rounding order of the library matmul
    np.testing.assert_allclose(out, out6, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lse6, rtol=0, atol=1e-14)


@pytest.mark.parametrize("q_len,n", [(5, 23), (33, 70)])  # a verify block, an extend chunk
def test_verify_row_equals_decode_over_prefix_plus_earlier_drafts(q_len, n):
    rng = np.random.default_rng(4)
    B, Hq, Hkv, D, P = 1, 4, 2, 16, 4
    q, kp, vp, table, kv = rand_case(rng, B, q_len, Hq, Hkv, D, P, [n])
    out, _ = oatt.verify_attention(q, kp, vp, table, kv, q_len, 0.25)
    L = n - q_len
    for i in range(q_len):
        d, _ = oatt.decode_attention(q[i], kp, vp, table[0], L + i + 1, 0.25)
        np.testing.assert_allclose(out[i], d, rtol=0, atol=1e-15)


def test_page_permutation_invariance():
    rng = np.random.default_rng(9)
    B, q_len, Hq, Hkv, D, P = 2, 2, 4, 2, 8, 4
    q, kp, vp, table, kv = rand_case(rng, B, q_len, Hq, Hkv, D, P, [11, 6])
    out, _ = oatt.verify_attention(q, kp, vp, table, kv, q_len, 0.3)
    perm = np.random.default_rng(1).permutation(kp.shape[0])
    inv = np.argsort(perm)
    kp2, vp2 = kp[perm], vp[perm]  # physical page perm[j] moves to slot j
    table2 = np.where(table >= 0, inv[np.maximum(table, 0)], -1)
    out2, _ = oatt.verify_attention(q, kp2, vp2, table2, kv, q_len, 0.3)
    np.testing.assert_array_equal(out, out2)


def test_merge_identity_over_arbitrary_partitions():
    rng = np.random.default_rng(12)
    B, q_len, Hq, Hkv, D, P = 2, 3, 4, 2, 8, 4
    lens = [30, 17]
    q, kp, vp, table, kv = rand_case(rng, B, q_len, Hq, Hkv, D, P, lens, scale=1.5)
    ref, ref_lse = oatt.verify_attention(q, kp, vp, table, kv, q_len, 0.4)
    for cuts in ([0, 30], [0, 8, 30], [0, 1, 2, 13, 16, 27, 30], [0, 16, 29, 30, 64]):
        parts = [oatt.attention_partial(q, kp, vp, table, kv, q_len, 0.4, lo, hi)
                 for lo, hi in zip(cuts[:-1], cuts[1:])]
        po = np.stack([p[0] for p in parts])
        pl = np.stack([p[1] for p in parts])
        out, lse = oatt.merge_partials(po, pl)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-13)


def test_merge_of_empty_partials():
    po = np.zeros((3, 2, 4))
    pl = np.full((3, 2), -np.inf)
    po[1, 0] = [1, 2, 3, 4]
    pl[1, 0] = 0.7
    out, lse = oatt.merge_partials(po, pl)
    np.testing.assert_array_equal(out[0], [1, 2, 3, 4])
    assert lse[0] == 0.7
    np.testing.assert_array_equal(out[1], 0)
    assert lse[1] == -np.inf


def test_merge_two_equal_halves_closed_form():
    # two partials with equal lse: out is their mean, lse + ln 2
    po = np.array([[[2.0, -4.0]], [[6.0, 0.0]]])
    pl = np.array([[1.25], [1.25]])
    out, lse = oatt.merge_partials(po, pl)
    np.testing.assert_allclose(out, [[4.0, -2.0]], atol=1e-15)
    np.testing.assert_allclose(lse, [1.25 + math.log(2)], atol=1e-15)


# ---------------------------------------------------------------------------
# FP8

def test_e4m3_table_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = ofp8.e4m3_decode(np.arange(256))
    finite = ~np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(ours), ~finite)
    np.testing.assert_array_equal(ours[finite], ref[finite])


def test_e4m3_special_values():
    v = ofp8.e4m3_value
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0
    assert v(0x38) == 1.0 and v(0x08) == 2.0 ** -6 and v(0x01) == 2.0 ** -9
    assert v(0x00) == 0.0 and math.copysign(1, v(0x80)) < 0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    # every finite E4M3 value is exactly representable in fp16
    vals = ofp8.e4m3_decode(np.arange(256))
    fin = vals[~np.isnan(vals)]
    np.testing.assert_array_equal(fin.astype(np.float16).astype(np.float64), fin)


def test_fp8_dequantized_attention_equals_fp64_attention_on_dequantized_values():
    rng = np.random.default_rng(5)
    P, q_len, Hq, Hkv, D = 4, 2, 2, 1, 128
    n = 10
    kc = rng.integers(0, 256, size=(4, Hkv, P, D)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(4, Hkv, P, D)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x10  # no NaN codes in valid data
    vc[(vc & 0x7F) == 0x7F] = 0x22
    ks = (rng.random((4, Hkv, P, D // 64)) * 0.01).astype(np.float16)
    vs = (rng.random((4, Hkv, P, D // 64)) * 0.01).astype(np.float16)
    table = np.array([[2, 0, 3]])
    q = rng.standard_normal((q_len, Hq, D)).astype(np.float16)
    out, _ = oatt.verify_attention(q, kc, vc, table, np.array([n]), q_len, 1 / 16, ks, vs)
    # dequantise by the formula, channel by channel, then use the fp16 path
    kd = np.zeros((4, Hkv, P, D))
    vd = np.zeros((4, Hkv, P, D))
    for p in range(4):
        for s in range(P):
            for c in range(D):
                kd[p, 0, s, c] = ofp8.e4m3_value(int(kc[p, 0, s, c])) * float(ks[p, 0, s, c // 64])
                vd[p, 0, s, c] = ofp8.e4m3_value(int(vc[p, 0, s, c])) * float(vs[p, 0, s, c // 64])
    ref, _ = oatt.verify_attention(q, kd, vd, table, np.array([n]), q_len, 1 / 16)
    np.testing.assert_array_equal(out, ref)


# ---------------------------------------------------------------------------
# greedy accept

def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _logits_with_argmax(am, V=64, seed=0):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((len(am), V)).astype(np.float32)
    lg[np.arange(len(am)), am] = 10.0
    return lg


@pytest.mark.parametrize("name", ["accept_worked_example.json", "accept_rejection_trace.json"])
def test_accept_printed_examples(golden_dir, name):
    g = _golden(golden_dir, name)
    q_len = g["q_len"]
    V = max(g["row_argmax"] + g["drafts"]) + 1
    lg = _logits_with_argmax(np.array(g["row_argmax"]), V=V)
    acc, bonus, am, new = oacc.greedy_accept(lg, np.array([g["drafts"]]), q_len, kv_lens=[100 + q_len])
    assert list(am) == g["row_argmax"]
    assert acc[0] == g["accept_len"] and bonus[0] == g["bonus"]
    assert new[0] == 100 + 1 + g["accept_len"]
    if "committed" in g:
        assert g["drafts"][:acc[0]] + [int(bonus[0])] == g["committed"]
    if "committed_stream_prefix" in g:
        assert [g["current_token"]] + (g["drafts"][:acc[0]] + [int(bonus[0])])[:1] == g["committed_stream_prefix"]
    a2, b2 = brute.greedy_accept(lg.tolist(), [g["drafts"]], q_len)
    assert (a2[0], b2[0]) == (g["accept_len"], g["bonus"])


def test_accept_planted_lengths_and_edges():
    rng = np.random.default_rng(3)
    q_len, V = 6, 50
    for a_star in range(q_len):
        targets = rng.integers(0, V, size=q_len)
        drafts = rng.integers(0, V, size=q_len - 1)
        drafts[:a_star] = targets[:a_star]
        if a_star < q_len - 1:
            drafts[a_star] = (targets[a_star] + 1) % V
        lg = _logits_with_argmax(targets, V=V, seed=a_star)
        acc, bonus, _, _ = oacc.greedy_accept(lg, drafts[None], q_len)
        assert acc[0] == a_star and bonus[0] == targets[a_star]
    # q = 1: nothing to accept, the bonus is plain greedy decode
    lg = _logits_with_argmax(np.array([17]), V=V)
    acc, bonus, _, _ = oacc.greedy_accept(lg, np.zeros((1, 0), np.int32), 1)
    assert acc[0] == 0 and bonus[0] == 17


def test_accept_ties_go_to_lowest_index():
    V = 1000
    lg = np.zeros((2, V), np.float32) - 1
    lg[0, [700, 3, 999]] = 5.0  # three-way tie
    lg[1, [998, 999]] = 2.0
    acc, bonus, am, _ = oacc.greedy_accept(lg, np.array([[3]]), 2)
    assert list(am) == [3, 998]
    assert acc[0] == 1 and bonus[0] == 998
    assert brute.argmax_first(lg[0].tolist()) == 3


def test_accept_batch_matches_brute_force():
    rng = np.random.default_rng(8)
    B, q_len, V = 5, 4, 30
    lg = rng.integers(-3, 4, size=(B * q_len, V)).astype(np.float32)  # many ties
    drafts = rng.integers(0, V, size=(B, q_len - 1))
    am = np.argmax(lg, axis=1)
    for b in range(B):  # make some prefixes match
        k = b % q_len
        drafts[b, :min(k, q_len - 1)] = am[b * q_len: b * q_len + min(k, q_len - 1)]
    acc, bonus, _, _ = oacc.greedy_accept(lg, drafts, q_len)
    a2, b2 = brute.greedy_accept(lg.tolist(), drafts.tolist(), q_len)
    assert list(acc) == a2 and list(bonus) == b2


# ---------------------------------------------------------------------------
# byte accounting printed on the pages

def test_kv_byte_pins(golden_dir):
    from long_context_gqa_amd.workloads import kv_bytes_per_token_head
    g = _golden(golden_dir, "kv_bytes.json")
    a = g["fixed_byte_test"]
    b = a["tokens"] * a["kv_heads"] * kv_bytes_per_token_head(a["head_dim"], "fp16")
    assert round(b / 1e6) == a["printed_megabytes"]
    c = g["kv_cache_per_rank"]
    fp16 = c["tokens"] * c["layers"] * c["kv_heads"] * kv_bytes_per_token_head(c["head_dim"], "fp16")
    assert round(fp16 / 2**20) == c["printed_mib_fp16"]
    fp8_data = c["tokens"] * c["layers"] * c["kv_heads"] * 2 * c["head_dim"]
    assert round(fp8_data / 2**20) == c["printed_mib_fp8_data"]


# ---------------------------------------------------------------------------
# the pins are sensitive: plant mistakes in copies of the oracle

def _shifted_causal(q, kp, vp, table, kv, q_len, sm):
    out, lse = oatt.verify_attention(q, kp, vp, table, kv, q_len, sm)
    # recompute each row with n_i + 1 visible keys where possible
    B = len(kv)
    for b in range(B):
        for i in range(q_len - 1):
            o2, l2 = oatt.decode_attention(q[b * q_len + i], kp, vp, table[b], kv[b] - q_len + i + 2, sm)
            out[b * q_len + i], lse[b * q_len + i] = o2, l2
    return out, lse


def _mutant_strided_gqa(q, kp, vp, table, kv, q_len, sm):
    Hq, Hkv = q.shape[1], kp.shape[1]
    G = Hq // Hkv
    # head h uses KV head h % Hkv instead of h // G
    perm = np.array([(h % Hkv) * G + (h // Hkv) for h in range(Hq)])
    out, lse = oatt.verify_attention(q[:, perm], kp, vp, table, kv, q_len, sm)
    inv = np.argsort(perm)
    return out[:, inv], lse[:, inv]


def _mutant_swapped_kv(q, kp, vp, table, kv, q_len, sm):
    return oatt.verify_attention(q, vp, kp, table, kv, q_len, sm)


def _mutant_no_scale(q, kp, vp, table, kv, q_len, sm):
    return oatt.verify_attention(q, kp, vp, table, kv, q_len, 1.0)


def _run_attention_pins(fn):
    """The attention pins above, parameterised by the implementation.
    Returns True when every pin holds."""
    try:
        rng = np.random.default_rng(7)
        q, kp, vp, table, kv = rand_case(rng, 2, 3, 4, 2, 8, 4, [7, 12])
        out, lse = fn(q, kp, vp, table, kv, 3, 1 / math.sqrt(8))
        bo, bl = brute.verify_attention(q.tolist(), kp.tolist(), vp.tolist(), table.tolist(),
                                        kv.tolist(), 3, 1 / math.sqrt(8))
        if not np.allclose(out, np.array(bo), rtol=0, atol=1e-12):
            return False
        L, q_len = 11, 3
        for i in range(q_len):
            for delta in (0, 1):
                t_star = L + i + delta
                q, kp, vp, table, kv, V = _probe_case(L, q_len, 4, 6, 2, 256, [t_star, 0])
                out, _ = fn(q, kp, vp, table, kv, q_len, 1.0 / 16)
                want = V[0][t_star] if delta == 0 else V[0][:L + i + 1].mean(axis=0)
                if not np.allclose(out[i, 0], want, atol=1e-12):
                    return False
                if not np.allclose(out[i, 5], V[1][0], atol=1e-12):
                    return False
        return True
    except (IndexError, ValueError):
        return False


def test_pins_catch_planted_mistakes():
    assert _run_attention_pins(oatt.verify_attention)
    for mutant in (_shifted_causal, _mutant_strided_gqa, _mutant_swapped_kv, _mutant_no_scale):
        assert not _run_attention_pins(mutant), mutant.__name__
