"""CPU oracle for the target-verify path — TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 implementations of what the verify step computes, written
from the pages' definitions:

  * ``attention.verify_attention`` — causal grouped-query attention of a
    verify block over a paged KV cache (fp16 or FP8 E4M3 + fp16 scales);
  * ``attention.merge_partials``   — combining split-KV partials (o, lse);
  * ``attention.verify_attention_ragged`` — the same with a different block
    width per request (rows packed request by request);
  * ``attention.verify_attention_window`` — the same over a leading sink
    prefix plus a sliding window of the newest positions;
  * ``accept.greedy_accept``       — argmax per row, longest matching draft
    prefix, bonus token, new cache length (``greedy_accept_ragged``: per-request
    widths);
  * ``block.prepare_block`` / ``block.append_kv`` — a block's packed rows,
    positions and cache slots, and writing its K/V into the reserved slots;
  * ``sampling.rejection_accept``  — stochastic acceptance: drafts kept by
    rejection sampling against target and draft probabilities, the final
    draw from the residual (or the last row);
  * ``topk.topk``                  — the k highest candidate logits of each row
    (value descending, lower index first on ties);
  * ``fp8.e4m3_decode``            — the OCP E4M3 value of each byte;
  * ``brute``                      — pure-Python loop versions for tiny inputs.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may
import this package. The library's compute path never does, and this package
imports nothing from the library.

Every function here is pinned by the ``-m "not gpu"`` tests against closed
forms, worked examples printed on the pages, library routines or brute force;
none is "parity unpinned".
"""
