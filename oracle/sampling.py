"""Stochastic acceptance of a verify block by rejection sampling — oracle,
test infrastructure only.

What is computed. At temperature zero the target keeps a draft token only
when it is the target's own choice ("Why the target output stayed the same",
page "MTP and DFlash2 at long context on XPU"); with sampling, acceptance
becomes rejection sampling against the target's and the draft's probabilities
(same passage; listed among the verify post-processing steps in section 1.1
of the page "DFlash -> dLLM self-spec, part 1"). The pages name the method
and no more, so the rule taken is the standard speculative-sampling one:

  p_j    = softmax(target logits of row j / T)   (the target's distribution
           for the token after t0, d_1, .., d_j)
  q_j    = the draft's distribution d_{j+1} was drawn from (given)
  for j = 0, 1, ..: keep d_{j+1} while  u_j * q_j(d_{j+1}) < p_j(d_{j+1})
           (u_j uniform on [0, 1): probability min(1, p/q))
  A      = the number kept
  token  = a draw, with u_final, from norm(max(p_A - q_A, 0)) if A < q_len-1
           (the first rejected row), else from p_{q_len-1} (every draft kept)
  new kv_len = kv_len - q_len + 1 + A

Readings (the pages are silent on each): the uniforms are inputs, one per
draft and one per request for the final draw; a draw from a distribution w
over the vocabulary by u is the smallest index v with w_0 + .. + w_v > u * sum(w)
(inverse CDF; ties cannot arise for u < 1); if the residual max(p - q, 0) is
zero everywhere (p = q at that row), the final draw is from p; temperature T > 0
scales the logits before the softmax, with no top-k/top-p filtering.
"""
from __future__ import annotations

import numpy as np


def _np(x, dtype=None):
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x, dtype=dtype)


def target_probs(logits_row, temperature):
    """softmax(logits / T) in float64."""
    z = _np(logits_row, np.float64) / float(temperature)
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def inverse_cdf(weights, u):
    """Smallest v with weights[0] + .. + weights[v] > u * sum(weights)."""
    w = _np(weights, np.float64)
    c = np.cumsum(w)
    v = int(np.searchsorted(c, u * c[-1], side="right"))
    return min(v, len(w) - 1)


def rejection_accept(logits, draft_ids, draft_probs, q_len, temperature, u_accept, u_final, kv_lens=None):
    """Returns (accept_len [B], token [B], new_kv_lens [B] or None).

    logits [B*q_len, V]; draft_ids [B, q_len-1]; draft_probs [B, q_len-1, V]
    (row j: the distribution d_{j+1} was drawn from); u_accept [B, q_len-1]
    and u_final [B] uniforms on [0, 1).
    """
    logits = _np(logits)
    B = logits.shape[0] // q_len
    ids = _np(draft_ids, np.int64).reshape(B, q_len - 1)
    dq = _np(draft_probs, np.float64)
    ua = _np(u_accept, np.float64).reshape(B, q_len - 1)
    uf = _np(u_final, np.float64)
    acc = np.zeros(B, dtype=np.int64)
    tok = np.zeros(B, dtype=np.int64)
    for b in range(B):
        a = 0
        while a < q_len - 1:
            d = ids[b, a]
            p = target_probs(logits[b * q_len + a], temperature)
            if ua[b, a] * dq[b, a, d] < p[d]:
                a += 1
            else:
                break
        acc[b] = a
        p = target_probs(logits[b * q_len + a], temperature)
        if a < q_len - 1:
            r = np.maximum(p - dq[b, a], 0.0)
            w = r if r.sum() > 0 else p
        else:
            w = p
        tok[b] = inverse_cdf(w, uf[b])
    new = None
    if kv_lens is not None:
        new = _np(kv_lens, np.int64) - q_len + 1 + acc
    return acc, tok, new
