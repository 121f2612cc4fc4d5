"""Greedy acceptance — oracle, test infrastructure only.

Rule (worked example "Why the target output stayed the same" on the page "MTP
and DFlash2 at long context on XPU"; verify table of section 1.1 and the
glossary entries "bonus token" and "accept length" on the page "DFlash ->
dLLM self-spec, part 1"): the block is [t0, d1, ..., d_{q-1}]; row j's logits
are the target's next-token distribution after t0, d1..dj, so draft d_{j+1}
is checked against argmax of row j. The accepted length A is the longest
prefix of drafts that all match; the bonus token is the target's choice at
the first mismatching row (row A), which is the last row when every draft
matches. The round commits A drafts plus the bonus, so the cache keeps
L + 1 + A positions (the page's commit_lens = accept_len + 1, section 1.6.1).

Argmax ties: the lowest index wins (numpy.argmax returns the first
occurrence); the pages test exact ties but do not print the rule.
"""
from __future__ import annotations

import numpy as np


def row_argmax(logits) -> np.ndarray:
    """Index of the largest value of every row, first occurrence on ties."""
    if hasattr(logits, "detach"):
        logits = logits.detach().cpu().numpy()
    return np.argmax(np.asarray(logits), axis=-1).astype(np.int64)


def accept_from_argmax(am, draft_ids, q_len, kv_lens=None):
    """Accepted length, bonus id and new cache length from per-row argmax.

    am        [B*q_len] target greedy choice of every verify row
    draft_ids [B, q_len-1]
    kv_lens   None, or [B] lengths including the block
    """
    am = np.asarray(am, dtype=np.int64)
    B = len(am) // q_len
    d = np.asarray(draft_ids, dtype=np.int64).reshape(B, max(q_len - 1, 0))
    acc = np.zeros(B, dtype=np.int64)
    bonus = np.zeros(B, dtype=np.int64)
    for b in range(B):
        a = 0
        while a < q_len - 1 and d[b, a] == am[b * q_len + a]:
            a += 1
        acc[b] = a
        bonus[b] = am[b * q_len + a]
    new_lens = None
    if kv_lens is not None:
        new_lens = np.asarray(kv_lens, dtype=np.int64) - q_len + 1 + acc
    return acc, bonus, new_lens


def greedy_accept(logits, draft_ids, q_len, kv_lens=None):
    """Returns (accept_len [B], bonus [B], argmax [B*q], new_kv_lens or None)."""
    am = row_argmax(logits)
    acc, bonus, new_lens = accept_from_argmax(am, draft_ids, q_len, kv_lens)
    return acc, bonus, am, new_lens


def greedy_accept_ragged(logits, block_ids, q_lens, q_start, kv_lens=None):
    """Greedy acceptance of blocks whose width differs per request.

    Request b's rows are q_start[b] .. q_start[b] + q_b - 1 of logits and of
    block_ids ([t0, d1, ..., d_{q_b-1}], packed as the block-preparation step
    lays them out), so the draft checked against row j is the block id one
    row later. Same rule as ``accept_from_argmax``: A is the longest prefix of
    drafts equal to the target's argmax of the previous row, the bonus is row
    A's argmax, and the cache keeps kv_len - q_b + 1 + A positions.

    Returns (accept_len [B], bonus [B], argmax [rows], new_kv_lens or None).
    """
    if hasattr(logits, "detach"):
        logits = logits.detach().cpu().numpy()
    am = np.argmax(np.asarray(logits), axis=-1).astype(np.int64)
    ids = np.asarray(block_ids.detach().cpu().numpy() if hasattr(block_ids, "detach") else block_ids,
                     dtype=np.int64)
    qn = np.asarray(q_lens, dtype=np.int64)
    qs = np.asarray(q_start, dtype=np.int64)
    B = len(qn)
    acc = np.zeros(B, dtype=np.int64)
    bonus = np.zeros(B, dtype=np.int64)
    for b in range(B):
        r0, qb = int(qs[b]), int(qn[b])
        a = 0
        while a < qb - 1 and ids[r0 + a + 1] == am[r0 + a]:
            a += 1
        acc[b] = a
        bonus[b] = am[r0 + a]
    new_lens = None
    if kv_lens is not None:
        new_lens = np.asarray(kv_lens, dtype=np.int64) - qn + 1 + acc
    return acc, bonus, am, new_lens
