"""Verify attention and split merge in float64 — oracle, test infrastructure only.

What is computed (plain definition, no blocking or reordering):

Verify block. A request with committed prefix L appends a block of q known
tokens (the current token and q-1 drafts); the target evaluates all q rows in
one causal pass, row j seeing the prefix and the block up to itself. This is
the worked example "Why the target output stayed the same" on the page "MTP
and DFlash2 at long context on XPU", and the verify table of section 1.1 on
the page "DFlash -> dLLM self-spec, part 1" (row j's logits come from
context + d1..dj). The same page (section 1.1) notes that the prefix KV
already exists and verify runs like a short extend over it; reading taken
here: the block's own K/V are already written into the paged cache, and
``kv_len`` counts them, so row i of request b sees the first
``kv_len[b] - q + i + 1`` cache positions.

Grouped-query attention with 24 query heads over 4 KV heads, head dimension
256 (PocketLLM page "Qwen3.8-27B-FP8", model specification table). Reading
taken: query head h uses KV head floor(h / (Hq / Hkv)) (contiguous groups).

Paged cache. Position t of request b lives in physical page
``page_table[b, t // P]`` at slot ``t % P`` (the request-to-token and token
pool indirection in the glossary of the self-spec page). Layout
[num_pages, Hkv, P, D].

FP8 mode (PocketLLM page, "Implemented execution path"): K and V are E4M3
bytes with one fp16 scale per token, per KV head and per 64-channel block; the
value of channel c is decode(code) * scale[c // 64].

For one row (request b, block row i, query head h):
    n  = kv_len[b] - q + i + 1
    s_t = sm_scale * sum_c Q[c] * K_t[c]           for t < n
    m  = max_t s_t,   w_t = exp(s_t - m),   l = sum_t w_t
    out = sum_t w_t V_t / l,   lse = m + ln l

Split merge (the compact online-softmax partials of the PocketLLM page's
split-context decode): partial s carries o_s (normalised over its own key
range) and lse_s; with LSE = ln sum_s exp(lse_s) over non-empty partials,
out = sum_s exp(lse_s - LSE) o_s. An empty partial has lse_s = -inf and
weight zero.
"""
from __future__ import annotations

import numpy as np

from . import fp8 as _fp8


def _as_np(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor on the CPU
        x = x.detach().cpu().numpy()
    return np.asarray(x)


def gather_kv(pages, scales, page_table_row, n, kv_head):
    """float64 rows [n, D] of one request and KV head, in position order."""
    P = pages.shape[2]
    npg = (n + P - 1) // P
    ids = np.asarray(page_table_row[:npg], dtype=np.int64)
    rows = pages[ids, kv_head].reshape(npg * P, pages.shape[3])[:n]
    if scales is None:
        return rows.astype(np.float64)
    sc = scales[ids, kv_head].reshape(npg * P, scales.shape[3])[:n]
    return _fp8.dequantize(rows, sc)


def verify_attention(q, k_pages, v_pages, page_table, kv_lens, q_len, sm_scale,
                     k_scales=None, v_scales=None, rows=None):
    """Exact causal GQA of every verify row.

    q           [B*q_len, Hq, D] fp16
    k_pages     [num_pages, Hkv, P, D] fp16, or uint8 E4M3 codes with scales
    v_pages     same layout as k_pages
    k_scales    None, or [num_pages, Hkv, P, D//64] fp16
    page_table  [B, max_pages] int32
    kv_lens     [B] int32, including the q_len block tokens
    rows        None for all, or an iterable of (b, kv_head) groups to compute
    Returns (out [B*q_len, Hq, D] float64, lse [B*q_len, Hq] float64); rows
    not requested are NaN.
    """
    q = _as_np(q)
    k_pages, v_pages = _as_np(k_pages), _as_np(v_pages)
    k_scales, v_scales = _as_np(k_scales), _as_np(v_scales)
    page_table, kv_lens = _as_np(page_table), _as_np(kv_lens)
    R, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    B = len(kv_lens)
    assert R == B * q_len and Hq % Hkv == 0
    G = Hq // Hkv
    out = np.full((R, Hq, D), np.nan)
    lse = np.full((R, Hq), np.nan)
    groups = [(b, g) for b in range(B) for g in range(Hkv)] if rows is None else list(rows)
    for b, g in groups:
        n_all = int(kv_lens[b])
        L = n_all - q_len
        K = gather_kv(k_pages, k_scales, page_table[b], n_all, g)
        V = gather_kv(v_pages, v_scales, page_table[b], n_all, g)
        Qg = q[b * q_len:(b + 1) * q_len, g * G:(g + 1) * G, :].astype(np.float64)  # [q, G, D]
        S = sm_scale * (Qg.reshape(q_len * G, D) @ K.T)  # [q*G, n]
        S = S.reshape(q_len, G, n_all)
        for i in range(q_len):
            n_i = L + i + 1
            s = S[i, :, :n_i]  # [G, n_i]
            m = s.max(axis=1, keepdims=True)
            w = np.exp(s - m)
            l = w.sum(axis=1, keepdims=True)
            out[b * q_len + i, g * G:(g + 1) * G] = (w @ V[:n_i]) / l
            lse[b * q_len + i, g * G:(g + 1) * G] = (m + np.log(l))[:, 0]
    return out, lse


def decode_attention(q_row, k_pages, v_pages, page_table_row, kv_len, sm_scale,
                     k_scales=None, v_scales=None):
    """Ordinary one-token decode: one query row [Hq, D] over the first kv_len
    cache positions. Same definition as a verify block of length 1."""
    q_row = _as_np(q_row)
    out, lse = verify_attention(q_row[None], k_pages, v_pages, _as_np(page_table_row)[None],
                                np.array([kv_len]), 1, sm_scale, k_scales, v_scales)
    return out[0], lse[0]


def attention_partial(q, k_pages, v_pages, page_table, kv_lens, q_len, sm_scale, t_lo, t_hi,
                      k_scales=None, v_scales=None):
    """Attention of every row restricted to key positions [t_lo, t_hi) (on top
    of the causal limit): the (o, lse) one split of the key range yields.
    Rows that see no key in the range get o = 0, lse = -inf."""
    q = _as_np(q)
    k_pages, v_pages = _as_np(k_pages), _as_np(v_pages)
    k_scales, v_scales = _as_np(k_scales), _as_np(v_scales)
    page_table, kv_lens = _as_np(page_table), _as_np(kv_lens)
    R, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    B = len(kv_lens)
    o = np.zeros((R, Hq, D))
    lse = np.full((R, Hq), -np.inf)
    for b in range(B):
        n_all = int(kv_lens[b])
        L = n_all - q_len
        for g in range(Hkv):
            K = gather_kv(k_pages, k_scales, page_table[b], n_all, g)
            V = gather_kv(v_pages, v_scales, page_table[b], n_all, g)
            for i in range(q_len):
                lo, hi = t_lo, min(t_hi, L + i + 1)
                if hi <= lo:
                    continue
                r = b * q_len + i
                Qh = q[r, g * G:(g + 1) * G].astype(np.float64)
                s = sm_scale * (Qh @ K[lo:hi].T)
                m = s.max(axis=1, keepdims=True)
                w = np.exp(s - m)
                l = w.sum(axis=1, keepdims=True)
                o[r, g * G:(g + 1) * G] = (w @ V[lo:hi]) / l
                lse[r, g * G:(g + 1) * G] = (m + np.log(l))[:, 0]
    return o, lse


def merge_partials(part_o, part_lse):
    """Combine split partials.

    part_o   [S, ..., D] — each partial normalised over its own key range
    part_lse [S, ...]    — log-sum-exp of its scaled logits, -inf if empty
    Returns (out [..., D], lse [...]) in float64; a row with every partial
    empty gets out = 0, lse = -inf.
    """
    po = _as_np(part_o).astype(np.float64)
    pl = _as_np(part_lse).astype(np.float64)
    mx = pl.max(axis=0)
    finite = np.isfinite(mx)
    ref = np.where(finite, mx, 0.0)
    w = np.where(np.isfinite(pl), np.exp(pl - ref[None]), 0.0)  # [S, ...]
    tot = w.sum(axis=0)
    safe = np.where(tot > 0, tot, 1.0)
    out = (w[..., None] * po).sum(axis=0) / safe[..., None]
    out = np.where(finite[..., None], out, 0.0)
    lse = np.where(finite, ref + np.log(safe), -np.inf)
    return out, lse


def verify_attention_ragged(q, k_pages, v_pages, page_table, kv_lens, q_lens, q_start, sm_scale,
                            k_scales=None, v_scales=None, groups=None):
    """Causal GQA of verify blocks whose width differs per request.

    Request b's block has q_b = q_lens[b] rows, stored at rows
    q_start[b] .. q_start[b] + q_b - 1 of q / out (the packing of the
    block-preparation step, see ``block.py``); kv_lens[b] counts the block.
    Row i of request b, query head h, sees the first kv_lens[b] - q_b + i + 1
    cache positions, exactly as in ``verify_attention``. Written per row, from
    the definition at the top of this module.

    Returns (out [rows, Hq, D], lse [rows, Hq]) in float64; rows of groups not
    requested are NaN.
    """
    q = _as_np(q)
    k_pages, v_pages = _as_np(k_pages), _as_np(v_pages)
    k_scales, v_scales = _as_np(k_scales), _as_np(v_scales)
    page_table, kv_lens = _as_np(page_table), _as_np(kv_lens)
    q_lens, q_start = _as_np(q_lens), _as_np(q_start)
    rows_total, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    B = len(kv_lens)
    out = np.full((rows_total, Hq, D), np.nan)
    lse = np.full((rows_total, Hq), np.nan)
    todo = [(b, g) for b in range(B) for g in range(Hkv)] if groups is None else list(groups)
    for b, g in todo:
        qb, n_all = int(q_lens[b]), int(kv_lens[b])
        K = gather_kv(k_pages, k_scales, page_table[b], n_all, g)
        V = gather_kv(v_pages, v_scales, page_table[b], n_all, g)
        for i in range(qb):
            r = int(q_start[b]) + i
            n = n_all - qb + i + 1
            for j in range(G):
                h = g * G + j
                s = sm_scale * (K[:n] @ q[r, h].astype(np.float64))  # [n]
                m = s.max()
                w = np.exp(s - m)
                l = w.sum()
                out[r, h] = (w @ V[:n]) / l
                lse[r, h] = m + np.log(l)
    return out, lse


def visible_keys(pos, window, sink):
    """Cache positions a row at position pos attends to with a sliding window
    of `window` positions (0: no window) and `sink` leading positions: every
    t <= pos with window == 0, or t < sink, or t > pos - window."""
    t = np.arange(pos + 1)
    if window == 0:
        return t
    return t[(t < sink) | (t > pos - window)]


def verify_attention_window(q, k_pages, v_pages, page_table, kv_lens, q_len, sm_scale, window, sink,
                            k_scales=None, v_scales=None, rows=None):
    """Verify attention with a leading sink prefix plus a sliding window.

    The PocketLLM page ("Implemented execution path"; "Validated performance",
    sparse experiments) describes an opt-in sparse mode that attends to the
    leading `sink` positions plus the newest `window` positions, without
    changing the KV-cache storage, and `window` = 0 is exact full attention.
    Reading taken: the window is counted per verify row and includes the row
    itself, so row i (position p = kv_len - q_len + i) sees t <= p with
    t < sink or t > p - window. Same layouts and return values as
    ``verify_attention``.
    """
    q = _as_np(q)
    k_pages, v_pages = _as_np(k_pages), _as_np(v_pages)
    k_scales, v_scales = _as_np(k_scales), _as_np(v_scales)
    page_table, kv_lens = _as_np(page_table), _as_np(kv_lens)
    R, Hq, D = q.shape
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    B = len(kv_lens)
    out = np.full((R, Hq, D), np.nan)
    lse = np.full((R, Hq), np.nan)
    groups = [(b, g) for b in range(B) for g in range(Hkv)] if rows is None else list(rows)
    for b, g in groups:
        n_all = int(kv_lens[b])
        K = gather_kv(k_pages, k_scales, page_table[b], n_all, g)
        V = gather_kv(v_pages, v_scales, page_table[b], n_all, g)
        for i in range(q_len):
            vis = visible_keys(n_all - q_len + i, window, sink)
            r = b * q_len + i
            for h in range(g * G, (g + 1) * G):
                s = sm_scale * (K[vis] @ q[r, h].astype(np.float64))
                m = s.max()
                w = np.exp(s - m)
                l = w.sum()
                out[r, h] = (w @ V[vis]) / l
                lse[r, h] = m + np.log(l)
    return out, lse
