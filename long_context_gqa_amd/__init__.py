"""Target-verify path of speculative decoding on MI355X (gfx950).

The compute lives in libsv.so (hand-written HIP kernels behind the C ABI of
include/sv.h); ``binding`` wraps its entry points with ctypes, and
``workloads`` draws seeded synthetic inputs.
"""
from . import binding, workloads  # noqa: F401
from .binding import (  # noqa: F401
    AcceptCall, PrepareCall, RaggedAcceptCall, RaggedVerifyCall, RejectionAcceptCall, SvError, TopkCall, VerifyCall, greedy_accept,
    make_params, sv_append_kv, sv_greedy_accept, sv_greedy_accept_ragged, sv_greedy_accept_workspace_bytes,
    sv_prepare_block, sv_rejection_accept, sv_topk_candidates, sv_verify_attention, sv_verify_attention_ragged, sv_verify_merge,
    sv_verify_plan,
    sv_verify_workspace_bytes, verify_attention,
)
