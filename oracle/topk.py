"""Top-k candidate selection over the vocabulary — oracle, test
infrastructure only.

What is computed. The draft side of DFlash2 takes, for every block position,
the 16 highest candidate logits of the target vocabulary head; under tensor
parallelism each rank first keeps its local top 16 and a second top 16 over
the gathered candidates gives the set an unsharded head would give (page "MTP
and DFlash2 at long context on XPU", the DFlash2 description; the selector
then scores transitions between adjacent candidate sets). The PocketLLM page
("Native MTP" flags table) splits each row's top 16 the same way and merges
with the identical comparator.

Reading taken (the pages print no order rule): candidates are ordered by
value, largest first, and equal values by the lower vocabulary index — the
tie rule of the greedy argmax. The output of a row is its first k entries in
that order: (index, value) pairs.
"""
from __future__ import annotations

import numpy as np


def topk_row(row, k):
    """(indices [k], values [k]) of one row, value descending, ties by lower index."""
    r = np.asarray(row)
    order = np.lexsort((np.arange(len(r)), -r.astype(np.float64)))
    top = order[:k]
    return top.astype(np.int64), r[top]


def topk(logits, k):
    """Row-wise top-k of logits [rows, V]: (indices [rows, k], values [rows, k])."""
    x = np.asarray(logits.detach().cpu().numpy() if hasattr(logits, "detach") else logits)
    idx = np.zeros((x.shape[0], k), dtype=np.int64)
    val = np.zeros((x.shape[0], k), dtype=x.dtype)
    for r in range(x.shape[0]):
        idx[r], val[r] = topk_row(x[r], k)
    return idx, val
