"""GPU parity of sv_rejection_accept (through the C ABI) against the float64
oracle: accepted length, drawn token and new cache length bit-exact. The
kernel decides in fp32 and the oracle in fp64, so the seeded uniforms are
redrawn (on the CPU, with the oracle's probabilities) until every decision is
at least a small relative margin away from its threshold; then both sides
must take the same decisions. Plus closed forms (draft = target, ids outside
the vocabulary) and the target-law property measured on many requests."""
import numpy as np
import pytest
import torch

from helpers import say
from long_context_gqa_amd import binding as B
from oracle import sampling as osm

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def make_case(Bn, q, V, T, seed, sigma=3.0, draft_noise=1.0, same=False):
    rng = np.random.default_rng(seed)
    logits = (rng.standard_normal((Bn * q, V)) * sigma).astype(np.float32)
    dq = np.zeros((Bn, max(q - 1, 0), V), dtype=np.float32)
    ids = np.zeros((Bn, max(q - 1, 0)), dtype=np.int32)
    for b in range(Bn):
        for j in range(q - 1):
            z = logits[b * q + j].astype(np.float64) / T
            if not same:
                z = z + rng.standard_normal(V) * draft_noise
            z -= z.max()
            w = np.exp(z)
            dq[b, j] = (w / w.sum()).astype(np.float32)
            ids[b, j] = rng.choice(V, p=dq[b, j].astype(np.float64) / dq[b, j].astype(np.float64).sum())
    ua = rng.random((Bn, max(q - 1, 0)))
    uf = rng.random(Bn)
    # keep every decision away from its threshold (relative margin)
    for b in range(Bn):
        for j in range(q - 1):
            p = osm.target_probs(logits[b * q + j], T)[ids[b, j]]
            qd = float(dq[b, j, ids[b, j]])
            while abs(ua[b, j] * qd - p) <= 1e-4 * max(p, ua[b, j] * qd):
                ua[b, j] = rng.random()
        A, _, _ = osm.rejection_accept(logits[b * q:(b + 1) * q], ids[b:b + 1], dq[b:b + 1], q, T, ua[b:b + 1],
                                       uf[b:b + 1])
        A = int(A[0])
        p = osm.target_probs(logits[b * q + A], T)
        w = np.maximum(p - dq[b, A], 0) if A < q - 1 else p
        if w.sum() <= 0:
            w = p
        c = np.cumsum(w)
        while True:
            t = uf[b] * c[-1]
            i = np.searchsorted(c, t)
            near = min(abs(c[max(i - 1, 0)] - t), abs(c[min(i, len(c) - 1)] - t))
            if near > 1e-5 * c[-1] and uf[b] < 1 - 1e-5:
                break
            uf[b] = rng.random()
    return logits, ids, dq, ua.astype(np.float32), uf.astype(np.float32)


def run_gpu(logits, ids, dq, q, T, ua, uf, kv):
    dev = "cuda"
    c = B.RejectionAcceptCall(torch.tensor(logits, device=dev), torch.tensor(ids, device=dev),
                              torch.tensor(dq, device=dev), q, T, torch.tensor(ua, device=dev),
                              torch.tensor(uf, device=dev), torch.tensor(kv, device=dev))
    acc, tok, new = c.run()
    torch.cuda.synchronize()
    return acc.cpu().numpy(), tok.cpu().numpy(), new.cpu().numpy()


@pytest.mark.parametrize("Bn,q,V,T", [
    (4, 8, 248_320, 1.0),     # the full vocabulary
    (4, 8, 248_320, 0.6),
    (8, 16, 50_000, 1.3),
    (3, 1, 248_320, 1.0),     # no drafts: a plain draw from row 0
    (5, 5, 1003, 0.9),        # a vocabulary that is not a multiple of 4
    (2, 3, 8192 * 3 + 5, 1.0),  # slices plus a short tail
])
def test_rejection_accept_matches_oracle(Bn, q, V, T):
    say(f"B={Bn} q={q} V={V} T={T}")
    logits, ids, dq, ua, uf = make_case(Bn, q, V, T, seed=Bn * 7 + q + V % 97)
    kv = np.array([1000 + 37 * b for b in range(Bn)], dtype=np.int32)
    acc, tok, new = run_gpu(logits, ids, dq, q, T, ua, uf, kv)
    ra, rt, rn = osm.rejection_accept(logits, ids, dq, q, T, ua.astype(np.float64), uf.astype(np.float64), kv)
    say(f"  accept {acc.tolist()}  tokens {tok.tolist()}")
    np.testing.assert_array_equal(acc, ra)
    np.testing.assert_array_equal(tok, rt)
    np.testing.assert_array_equal(new, rn)


def test_draft_equal_to_target_keeps_every_draft():
    Bn, q, V, T = 4, 8, 20_000, 1.0
    logits, ids, dq, ua, uf = make_case(Bn, q, V, T, seed=11, same=True)
    # same distribution (up to fp32 rounding of q): keep when u * q < p,
    # so only u well below 1 is certain; the margins above already hold
    ua = np.minimum(ua, 0.99).astype(np.float32)
    acc, tok, new = run_gpu(logits, ids, dq, q, T, ua, uf, np.full(Bn, 500, dtype=np.int32))
    np.testing.assert_array_equal(acc, q - 1)
    ra, rt, _ = osm.rejection_accept(logits, ids, dq, q, T, ua.astype(np.float64), uf.astype(np.float64))
    np.testing.assert_array_equal(tok, rt)


def test_ids_outside_the_vocabulary_are_rejected():
    Bn, q, V, T = 3, 6, 5000, 1.0
    logits, ids, dq, ua, uf = make_case(Bn, q, V, T, seed=12, same=True)
    ua = np.minimum(ua, 0.99).astype(np.float32)
    ids[0, 2] = V          # past the end
    ids[1, 0] = -1         # negative
    acc, tok, _ = run_gpu(logits, ids, dq, q, T, ua, uf, np.full(Bn, 500, dtype=np.int32))
    assert acc.tolist() == [2, 0, q - 1]


def test_first_committed_token_follows_the_target_law():
    # many requests with one draft each over the same target row and draft
    # distribution: the first committed token (the draft if kept, else the
    # draw) is distributed as p = softmax(row / T), whatever q is
    Bn, q, V, T = 8192, 2, 64, 0.8
    rng = np.random.default_rng(21)
    row = (rng.standard_normal(V) * 2).astype(np.float32)
    qd = rng.dirichlet(np.ones(V)).astype(np.float32)
    logits = np.tile(row, (Bn * q, 1))
    dq = np.tile(qd, (Bn, 1, 1))
    ids = rng.choice(V, size=(Bn, 1), p=qd.astype(np.float64) / qd.astype(np.float64).sum()).astype(np.int32)
    ua = rng.random((Bn, 1)).astype(np.float32)
    uf = rng.random(Bn).astype(np.float32)
    acc, tok, _ = run_gpu(logits, ids, dq, q, T, ua, uf, np.full(Bn, 10, dtype=np.int32))
    first = np.where(acc == 1, ids[:, 0], tok)
    freq = np.bincount(first, minlength=V) / Bn
    p = osm.target_probs(row, T)
    sd = np.sqrt(p * (1 - p) / Bn)
    z = np.abs(freq - p) / np.maximum(sd, 1e-12)
    say(f"  max |freq - p| {np.abs(freq - p).max():.4f}, max z {z.max():.2f}")
    assert z.max() < 5.0
    # and with the acceptance ratio inverted the law is visibly wrong (the
    # same statistic on the oracle's planted mistake, CPU side)
    assert np.abs(qd - p).max() > 0.02


@pytest.mark.parametrize("wl_id", [4, 3])
def test_full_size_workload_inputs(wl_id):
    # the workload's logits (32 x 16 rows or 1 x 8 of 248,320) with the
    # generator's draft distributions and uniforms, unadjusted: every request
    # must match the oracle unless its deciding comparison is borderline
    from long_context_gqa_amd import workloads as W
    wl = W.WORKLOADS[wl_id]
    acc_in = W.make_accept_inputs(wl, device="cuda")
    si = W.make_sampling_inputs(wl, device="cuda")
    kv = torch.full((wl.batch,), 5000, dtype=torch.int32, device="cuda")
    c = B.RejectionAcceptCall(acc_in.logits, si.draft_ids, si.draft_probs, wl.q_len, 1.0, si.u_accept, si.u_final, kv)
    acc, tok, new = [t.cpu().numpy() for t in c.run()]
    torch.cuda.synchronize()
    lg = acc_in.logits.cpu().numpy()
    ids, dq = si.draft_ids.cpu().numpy(), si.draft_probs.cpu().numpy()
    ua, uf = si.u_accept.cpu().numpy().astype(np.float64), si.u_final.cpu().numpy().astype(np.float64)
    ra, rt, rn = osm.rejection_accept(lg, ids, dq, wl.q_len, 1.0, ua, uf, kv.cpu().numpy())
    q = wl.q_len
    say(f"  accept lengths {acc.tolist()[:16]}")
    for b in range(wl.batch):
        if acc[b] == ra[b] and tok[b] == rt[b]:
            continue
        if acc[b] != ra[b]:
            # the accepted lengths differ: the acceptance test of the first
            # row where they part must sit within 1e-4 of its threshold
            j = min(acc[b], ra[b])
            p = osm.target_probs(lg[b * q + j], 1.0)
            d = ids[b, j]
            margin = abs(ua[b, j] * dq[b, j, d] - p[d]) / max(p[d], 1e-30)
            bound = 1e-4
        else:
            # same length, another token: the final draw (from the residual
            # at the first rejected row, or from p when every draft is kept)
            # must have a cumulative weight within 1e-5 of its target
            A = int(acc[b])
            p = osm.target_probs(lg[b * q + A], 1.0)
            w = np.maximum(p - dq[b, A].astype(np.float64), 0.0) if A < q - 1 else p
            if not (w > 0).any():
                w = p
            cs = np.cumsum(w)
            margin = np.abs(cs - uf[b] * cs[-1]).min() / cs[-1]
            bound = 1e-5
        say(f"  request {b}: gpu ({acc[b]}, {tok[b]}) oracle ({ra[b]}, {rt[b]}), margin {margin:.2e}")
        assert margin < bound
    np.testing.assert_array_equal(new - acc, rn - ra)
