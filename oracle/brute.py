"""Pure-Python loop versions for tiny inputs — oracle, test infrastructure only.

The "small loop references" idea of the page "MTP and DFlash2 at long
context on XPU" (section on the DFlash2 selector): plain loops over scalars,
compared against the vectorised path. Sums use math.fsum (exactly rounded),
exponentials math.exp. Inputs are nested lists / scalars; the definitions are
the ones in ``oracle.attention`` and ``oracle.accept``.
"""
from __future__ import annotations

import math


def attention_row(qvec, keys, values, sm_scale):
    """Softmax attention of one query over the given key/value rows."""
    s = [sm_scale * math.fsum(a * b for a, b in zip(qvec, k)) for k in keys]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    l = math.fsum(w)
    d = len(values[0])
    out = [math.fsum(w[t] * values[t][c] for t in range(len(values))) / l for c in range(d)]
    return out, m + math.log(l)


def verify_attention(q, k_pages, v_pages, page_table, kv_lens, q_len, sm_scale):
    """q[r][h][c], k_pages[page][g][slot][c] as nested lists (already real
    numbers). Returns out[r][h][c], lse[r][h]."""
    B = len(kv_lens)
    Hq = len(q[0])
    Hkv = len(k_pages[0])
    G = Hq // Hkv
    P = len(k_pages[0][0])
    out = [[None] * Hq for _ in range(B * q_len)]
    lse = [[None] * Hq for _ in range(B * q_len)]
    for b in range(B):
        L = kv_lens[b] - q_len
        for i in range(q_len):
            r = b * q_len + i
            n = L + i + 1
            for h in range(Hq):
                g = h // G
                keys = [k_pages[page_table[b][t // P]][g][t % P] for t in range(n)]
                vals = [v_pages[page_table[b][t // P]][g][t % P] for t in range(n)]
                out[r][h], lse[r][h] = attention_row(q[r][h], keys, vals, sm_scale)
    return out, lse


def argmax_first(row):
    best, bi = row[0], 0
    for i, x in enumerate(row):
        if x > best:
            best, bi = x, i
    return bi


def greedy_accept(logit_rows, drafts, q_len):
    """logit_rows[b*q+j][v], drafts[b][j]. Returns (accept, bonus) lists."""
    B = len(logit_rows) // q_len
    acc, bonus = [], []
    for b in range(B):
        am = [argmax_first(logit_rows[b * q_len + j]) for j in range(q_len)]
        a = 0
        while a < q_len - 1 and drafts[b][a] == am[a]:
            a += 1
        acc.append(a)
        bonus.append(am[a])
    return acc, bonus
