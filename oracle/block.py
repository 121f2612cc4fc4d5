"""Preparing a verify block and appending its K/V — oracle, test infrastructure only.

What is computed. The self-spec page ("DFlash -> dLLM self-spec, part 1")
lists, in section 1.3.3, a fused block-preparation step that yields a
round's block token ids, positions and cache locations in one pass, and a
fused accept step that yields accept length, bonus and new sequence lengths.
Section 1.3.2 ("KV over-allocation") reserves the slots of the coming block
ahead of time, so the worker finds each block token's cache location straight
from the request-to-token table. The verify width may differ per request:
the PocketLLM page ("Native MTP" / DFlash2 table) verifies an adaptive number
of rows per round, and DSpark (section 1.7.2 of the self-spec page) lets a
scheduler pick each request's verify length.

For request b with committed length L_b = seq_lens[b] and block width
q_b = q_lens[b]:

    q_start[b]  = q_0 + ... + q_{b-1}     (the block rows of all requests, packed)
    position    = L_b + i                 (i < q_b)
    cache slot  = page_table[b, position // P] * P + position % P
    kv_len_out  = L_b + q_b               (the cache as the verify pass sees it)
    block ids   = [last_token[b], d_1, ..., d_{q_b - 1}]

Appending writes row q_start[b] + i of the new K and V (every KV head) into
its cache slot: pages[slot // P, h, slot % P, :] = new[row, h, :].

With an FP8 cache the appended rows are quantised first (oracle.fp8,
quantize_rows): E4M3 codes into the pages and one fp16 scale per token, KV
head and 64-channel block into the scale pages.

Readings taken (the pages name the steps but not their data layout): rows are
packed request by request; drafts come padded as [B, max_q - 1] and the block
ids come out packed like the rows; the cache slot is the flat index
page * P + slot of the pool.
"""
from __future__ import annotations

import numpy as np


def _np(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x)


def prepare_block(seq_lens, q_lens, page_table, page_size, last_tokens=None, drafts=None):
    """Returns dict(q_start [B+1], positions [rows], cache_slot [rows],
    kv_lens_out [B], block_ids [rows] or None); rows = sum of q_lens."""
    L = _np(seq_lens).astype(np.int64)
    qn = _np(q_lens).astype(np.int64)
    pt = _np(page_table).astype(np.int64)
    B = len(L)
    q_start = np.zeros(B + 1, dtype=np.int64)
    for b in range(B):
        q_start[b + 1] = q_start[b] + qn[b]
    rows = int(q_start[B])
    positions = np.zeros(rows, dtype=np.int64)
    slots = np.zeros(rows, dtype=np.int64)
    ids = None if last_tokens is None else np.zeros(rows, dtype=np.int64)
    d = None if drafts is None else _np(drafts).astype(np.int64)
    lt = None if last_tokens is None else _np(last_tokens).astype(np.int64)
    for b in range(B):
        for i in range(int(qn[b])):
            r = int(q_start[b]) + i
            pos = int(L[b]) + i
            positions[r] = pos
            slots[r] = pt[b, pos // page_size] * page_size + pos % page_size
            if ids is not None:
                ids[r] = lt[b] if i == 0 else d[b, i - 1]
    return dict(q_start=q_start, positions=positions, cache_slot=slots, kv_lens_out=L + qn,
                block_ids=ids)


def append_kv(pages, cache_slot, new_rows):
    """A copy of pages [num_pages, Hkv, P, D] with new_rows [rows, Hkv, D]
    written at the given flat cache slots."""
    out = _np(pages).copy()
    slots = _np(cache_slot).astype(np.int64)
    new = _np(new_rows)
    P = out.shape[2]
    for r, s in enumerate(slots):
        out[s // P, :, s % P, :] = new[r]
    return out


def append_kv_fp8(pages, scales, cache_slot, new_rows):
    """Copies of FP8 pages [num_pages, Hkv, P, D] (E4M3 bytes) and scales
    [num_pages, Hkv, P, D//64] (fp16) with new_rows [rows, Hkv, D] quantised
    (oracle.fp8.quantize_rows) and written at the given flat cache slots."""
    from oracle.fp8 import quantize_rows
    out, osc = _np(pages).copy(), _np(scales).copy()
    slots = _np(cache_slot).astype(np.int64)
    codes, sc = quantize_rows(_np(new_rows))
    P = out.shape[2]
    for r, s in enumerate(slots):
        out[s // P, :, s % P, :] = codes[r]
        osc[s // P, :, s % P, :] = sc[r]
    return out, osc
