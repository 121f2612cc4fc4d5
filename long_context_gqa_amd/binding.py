"""ctypes binding of libsv.so (include/sv.h): argument marshalling only.

Every function here has the name of the C entry point it wraps, takes torch
tensors that live on the GPU (torch is used only to own device memory and to
name the stream) and passes their pointers through. Nothing here computes a
step of the verify path; there is no fallback: if the library is missing the
call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsv.so")

SV_OK, SV_ERR_INVALID_ARGUMENT, SV_ERR_UNSUPPORTED, SV_ERR_WORKSPACE_TOO_SMALL, SV_ERR_HIP = range(5)
SV_KV_FP16, SV_KV_FP8_E4M3 = 0, 1
SV_FLAG_KV_LEN_ABOVE_BOUND, SV_FLAG_KV_LEN_BELOW_BLOCK, SV_FLAG_PAGE_ID_OUT_OF_RANGE = 1, 2, 4
SV_FLAG_BAD_BLOCK_WIDTH, SV_FLAG_WORKSPACE_NOT_ZERO = 8, 0x10
SV_VERIFY_CLAIMED_WORK = 0x1

EXPORTED = (
    "sv_verify_workspace_bytes", "sv_verify_plan", "sv_verify_attention", "sv_verify_merge",
    "sv_greedy_accept_workspace_bytes", "sv_greedy_accept", "sv_verify_attention_ragged",
    "sv_greedy_accept_ragged", "sv_prepare_block", "sv_append_kv", "sv_append_kv_fp8",
    "sv_rejection_accept_workspace_bytes",
    "sv_rejection_accept", "sv_topk_candidates_workspace_bytes", "sv_topk_candidates", "sv_status_string",
    "sv_last_error", "sv_version", "sv_verify_scratch_bytes", "sv_verify_attention_noalloc",
    "sv_verify_plan_kernel",
)
SV_KERNEL_ROW_TILES, SV_KERNEL_TWO_HALVES = 0, 1


class SvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


class SvVerifyParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_req", ctypes.c_int32),
        ("max_kv_len", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int),
        ("sm_scale", ctypes.c_float),
        ("num_splits", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("sink", ctypes.c_int32),
        ("options", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libsv.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m long_context_gqa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32, f32p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p
        P = ctypes.POINTER(SvVerifyParams)
        L.sv_verify_workspace_bytes.argtypes = [P]
        L.sv_verify_workspace_bytes.restype = sz
        L.sv_verify_plan.argtypes = [P, ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.sv_verify_plan.restype = ctypes.c_int
        L.sv_verify_plan_kernel.argtypes = [P, ctypes.POINTER(i32)]
        L.sv_verify_plan_kernel.restype = ctypes.c_int
        L.sv_verify_attention.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, f32p, vp, sz, vp, vp]
        L.sv_verify_attention.restype = ctypes.c_int
        L.sv_verify_scratch_bytes.argtypes = []
        L.sv_verify_scratch_bytes.restype = sz
        L.sv_verify_attention_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, f32p, vp, vp]
        L.sv_verify_attention_noalloc.restype = ctypes.c_int
        L.sv_verify_merge.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp]
        L.sv_verify_merge.restype = ctypes.c_int
        L.sv_greedy_accept_workspace_bytes.argtypes = [i32, i32, i32]
        L.sv_greedy_accept_workspace_bytes.restype = sz
        L.sv_greedy_accept.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.sv_greedy_accept.restype = ctypes.c_int
        L.sv_verify_attention_ragged.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, f32p, vp, sz, vp, vp]
        L.sv_verify_attention_ragged.restype = ctypes.c_int
        L.sv_greedy_accept_ragged.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp, vp]
        L.sv_greedy_accept_ragged.restype = ctypes.c_int
        L.sv_prepare_block.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.sv_prepare_block.restype = ctypes.c_int
        L.sv_append_kv.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, ctypes.c_int, vp, vp, vp, vp]
        L.sv_append_kv.restype = ctypes.c_int
        L.sv_append_kv_fp8.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.sv_append_kv_fp8.restype = ctypes.c_int
        L.sv_rejection_accept_workspace_bytes.argtypes = [i32, i32, i32]
        L.sv_rejection_accept_workspace_bytes.restype = sz
        L.sv_rejection_accept.argtypes = [vp, vp, vp, i32, i32, i32, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, sz,
                                          vp]
        L.sv_rejection_accept.restype = ctypes.c_int
        L.sv_topk_candidates_workspace_bytes.argtypes = [i32, i32, i32]
        L.sv_topk_candidates_workspace_bytes.restype = sz
        L.sv_topk_candidates.argtypes = [vp, i32, i32, i32, vp, vp, vp, sz, vp]
        L.sv_topk_candidates.restype = ctypes.c_int
        L.sv_status_string.argtypes = [ctypes.c_int]
        L.sv_status_string.restype = ctypes.c_char_p
        L.sv_last_error.argtypes = []
        L.sv_last_error.restype = ctypes.c_char_p
        L.sv_version.argtypes = []
        L.sv_version.restype = i32
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("device tensors only")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != SV_OK:
        raise SvError(status, lib().sv_last_error().decode())


def make_params(batch, q_len, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                max_pages_per_req, max_kv_len, kv_dtype=SV_KV_FP16, sm_scale=None, num_splits=0, window=0,
                sink=0, options=0):
    if sm_scale is None:
        sm_scale = head_dim ** -0.5
    return SvVerifyParams(batch, q_len, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                          max_pages_per_req, max_kv_len, kv_dtype, sm_scale, num_splits, window, sink, options)


def sv_verify_workspace_bytes(p: SvVerifyParams) -> int:
    return int(lib().sv_verify_workspace_bytes(ctypes.byref(p)))


def sv_verify_plan(p: SvVerifyParams) -> tuple[int, int]:
    s, c = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().sv_verify_plan(ctypes.byref(p), ctypes.byref(s), ctypes.byref(c)))
    return s.value, c.value


def sv_verify_plan_kernel(p: SvVerifyParams) -> int:
    """SV_KERNEL_ROW_TILES or SV_KERNEL_TWO_HALVES: the kernel the plan launches."""
    k = ctypes.c_int32()
    _check(lib().sv_verify_plan_kernel(ctypes.byref(p), ctypes.byref(k)))
    return k.value


def sv_verify_attention(p: SvVerifyParams, q, k_pages, v_pages, k_scales, v_scales, page_table, kv_lens,
                        out, out_lse=None, workspace=None, status_flags=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().sv_verify_attention(ctypes.byref(p), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scales),
                                      _ptr(v_scales), _ptr(page_table), _ptr(kv_lens), _ptr(out),
                                      _ptr(out_lse), _ptr(workspace), ws_bytes, _ptr(status_flags),
                                      _stream(stream)))


def sv_verify_scratch_bytes() -> int:
    return int(lib().sv_verify_scratch_bytes())


def sv_verify_attention_noalloc(p: SvVerifyParams, q, k_pages, v_pages, k_scales, v_scales, page_table, kv_lens,
                                out, out_lse=None, status_flags=None, stream=None):
    _check(lib().sv_verify_attention_noalloc(ctypes.byref(p), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                             _ptr(k_scales), _ptr(v_scales), _ptr(page_table), _ptr(kv_lens),
                                             _ptr(out), _ptr(out_lse), _ptr(status_flags), _stream(stream)))


def sv_verify_merge(part_o, part_lse, out, out_lse=None, stream=None):
    S, R, H, D = part_o.shape
    _check(lib().sv_verify_merge(_ptr(part_o), _ptr(part_lse), S, R, H, D, _ptr(out), _ptr(out_lse),
                                 _stream(stream)))


def sv_greedy_accept_workspace_bytes(batch: int, q_len: int, vocab: int) -> int:
    return int(lib().sv_greedy_accept_workspace_bytes(batch, q_len, vocab))


def sv_greedy_accept(logits, draft_ids, batch, q_len, vocab, accept_len, bonus_ids, argmax_ids=None,
                     kv_lens_in=None, kv_lens_out=None, workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().sv_greedy_accept(_ptr(logits), _ptr(draft_ids) if q_len > 1 else None, batch, q_len, vocab,
                                  _ptr(accept_len), _ptr(bonus_ids), _ptr(argmax_ids), _ptr(kv_lens_in),
                                  _ptr(kv_lens_out), _ptr(workspace), ws_bytes, _stream(stream)))


def sv_verify_attention_ragged(p: SvVerifyParams, q_start, q, k_pages, v_pages, k_scales, v_scales, page_table,
                               kv_lens, out, out_lse=None, workspace=None, status_flags=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().sv_verify_attention_ragged(ctypes.byref(p), _ptr(q_start), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                             _ptr(k_scales), _ptr(v_scales), _ptr(page_table), _ptr(kv_lens),
                                             _ptr(out), _ptr(out_lse), _ptr(workspace), ws_bytes,
                                             _ptr(status_flags), _stream(stream)))


def sv_greedy_accept_ragged(logits, block_ids, q_start, batch, max_q_len, vocab, accept_len, bonus_ids,
                            argmax_ids=None, kv_lens_in=None, kv_lens_out=None, workspace=None, status_flags=None,
                            stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().sv_greedy_accept_ragged(_ptr(logits), _ptr(block_ids), _ptr(q_start), batch, max_q_len, vocab,
                                         _ptr(accept_len), _ptr(bonus_ids), _ptr(argmax_ids), _ptr(kv_lens_in),
                                         _ptr(kv_lens_out), _ptr(workspace), ws_bytes, _ptr(status_flags),
                                         _stream(stream)))


def sv_prepare_block(seq_lens, q_lens, page_table, batch, max_q_len, page_size, num_pages, q_start, cache_slot,
                     positions=None, kv_lens_out=None, last_tokens=None, draft_ids=None, block_ids=None,
                     status_flags=None, stream=None):
    _check(lib().sv_prepare_block(_ptr(seq_lens), _ptr(q_lens), _ptr(page_table), batch, max_q_len,
                                  page_table.shape[1], page_size, num_pages, _ptr(last_tokens), _ptr(draft_ids),
                                  _ptr(q_start), _ptr(positions), _ptr(cache_slot), _ptr(kv_lens_out),
                                  _ptr(block_ids), _ptr(status_flags), _stream(stream)))


def sv_append_kv(new_k, new_v, cache_slot, q_start, batch, max_rows, k_pages, v_pages, status_flags=None,
                 stream=None):
    num_pages, Hkv, P, D = k_pages.shape
    _check(lib().sv_append_kv(_ptr(new_k), _ptr(new_v), _ptr(cache_slot), _ptr(q_start), batch, max_rows, Hkv, D, P,
                              num_pages, SV_KV_FP16 if k_pages.dtype == torch.float16 else SV_KV_FP8_E4M3,
                              _ptr(k_pages), _ptr(v_pages), _ptr(status_flags), _stream(stream)))


def sv_append_kv_fp8(new_k, new_v, cache_slot, q_start, batch, max_rows, k_pages, v_pages, k_scales, v_scales,
                     status_flags=None, stream=None):
    """Quantise new fp16 K/V rows per 64-channel block into E4M3 pages (uint8)
    and their fp16 scale pages at the rows' cache slots."""
    num_pages, Hkv, P, D = k_pages.shape
    _check(lib().sv_append_kv_fp8(_ptr(new_k), _ptr(new_v), _ptr(cache_slot), _ptr(q_start), batch, max_rows, Hkv, D,
                                  P, num_pages, _ptr(k_pages), _ptr(v_pages), _ptr(k_scales), _ptr(v_scales),
                                  _ptr(status_flags), _stream(stream)))


def sv_rejection_accept_workspace_bytes(batch: int, q_len: int, vocab: int) -> int:
    return int(lib().sv_rejection_accept_workspace_bytes(batch, q_len, vocab))


def sv_rejection_accept(logits, draft_ids, draft_probs, batch, q_len, vocab, temperature, u_accept, u_final,
                        accept_len, token_ids, kv_lens_in=None, kv_lens_out=None, workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().sv_rejection_accept(_ptr(logits), _ptr(draft_ids), _ptr(draft_probs), batch, q_len, vocab,
                                     float(temperature), _ptr(u_accept), _ptr(u_final), _ptr(accept_len),
                                     _ptr(token_ids), _ptr(kv_lens_in), _ptr(kv_lens_out), _ptr(workspace), ws_bytes,
                                     _stream(stream)))


def sv_topk_candidates_workspace_bytes(rows: int, vocab: int, k: int) -> int:
    return int(lib().sv_topk_candidates_workspace_bytes(rows, vocab, k))


def sv_topk_candidates(logits, k, out_ids, out_values, workspace, stream=None):
    rows, vocab = logits.shape
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().sv_topk_candidates(_ptr(logits), rows, vocab, k, _ptr(out_ids), _ptr(out_values), _ptr(workspace),
                                    ws_bytes, _stream(stream)))


def sv_version() -> int:
    return int(lib().sv_version())


# ---------------------------------------------------------------------------
# Convenience wrappers: allocate outputs and workspace with torch, then call
# the entry points above. Still marshalling only.

class VerifyCall:
    """Device buffers and parameters of one verify-attention call, reusable
    across launches (the benchmark times ``run`` in a loop)."""

    def __init__(self, q, k_pages, v_pages, page_table, kv_lens, q_len, max_kv_len,
                 k_scales=None, v_scales=None, sm_scale=None, num_splits=0, with_lse=True, window=0, sink=0,
                 claim=False):
        dev = q.device
        B = kv_lens.shape[0]
        Hq, D = q.shape[1], q.shape[2]
        Hkv, P = k_pages.shape[1], k_pages.shape[2]
        dtype = SV_KV_FP8_E4M3 if k_pages.dtype == torch.uint8 else SV_KV_FP16
        self.params = make_params(B, q_len, Hq, Hkv, D, P, k_pages.shape[0], page_table.shape[1],
                                  max_kv_len, dtype, sm_scale, num_splits, window, sink,
                                  SV_VERIFY_CLAIMED_WORK if claim else 0)
        self.inputs = (q, k_pages, v_pages, k_scales, v_scales, page_table, kv_lens)
        self.out = torch.empty_like(q)
        self.out_lse = torch.empty((q.shape[0], Hq), dtype=torch.float32, device=dev) if with_lse else None
        nbytes = sv_verify_workspace_bytes(self.params)
        # zero-filled once: its first 32 KB are work counters every call leaves at zero
        self.workspace = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
        self.flags = torch.zeros(1, dtype=torch.int32, device=dev)
        self.splits, self.chunk = sv_verify_plan(self.params)
        self.kernel = sv_verify_plan_kernel(self.params)

    def run(self, stream=None):
        sv_verify_attention(self.params, *self.inputs, self.out, self.out_lse, self.workspace, self.flags,
                            stream)
        return self.out, self.out_lse


def verify_attention(q, k_pages, v_pages, page_table, kv_lens, q_len, max_kv_len=None, k_scales=None,
                     v_scales=None, sm_scale=None, num_splits=0, window=0, sink=0, claim=False):
    """One verify-attention call; returns (out fp16, lse fp32, status flags)."""
    if max_kv_len is None:
        raise ValueError("max_kv_len (a host upper bound) is required")
    c = VerifyCall(q, k_pages, v_pages, page_table, kv_lens, q_len, max_kv_len, k_scales, v_scales, sm_scale,
                   num_splits, window=window, sink=sink, claim=claim)
    c.run()
    return c.out, c.out_lse, c.flags


class AcceptCall:
    def __init__(self, logits, draft_ids, q_len, kv_lens=None, with_argmax=True):
        dev = logits.device
        self.batch = logits.shape[0] // q_len
        self.q_len, self.vocab = q_len, logits.shape[1]
        self.logits, self.draft_ids = logits, draft_ids
        self.accept_len = torch.empty(self.batch, dtype=torch.int32, device=dev)
        self.bonus = torch.empty(self.batch, dtype=torch.int32, device=dev)
        self.argmax = torch.empty(logits.shape[0], dtype=torch.int32, device=dev) if with_argmax else None
        self.kv_in = kv_lens
        self.kv_out = torch.empty_like(kv_lens) if kv_lens is not None else None
        nbytes = sv_greedy_accept_workspace_bytes(self.batch, q_len, self.vocab)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)

    def run(self, stream=None):
        sv_greedy_accept(self.logits, self.draft_ids, self.batch, self.q_len, self.vocab, self.accept_len,
                         self.bonus, self.argmax, self.kv_in, self.kv_out, self.workspace, stream)
        return self.accept_len, self.bonus, self.argmax, self.kv_out


def greedy_accept(logits, draft_ids, q_len, kv_lens=None):
    c = AcceptCall(logits, draft_ids, q_len, kv_lens)
    return c.run()


# ---------------------------------------------------------------------------
# Blocks of a width per request

class RaggedVerifyCall:
    """Device buffers of one verify-attention call over packed blocks of
    different widths (rows of request b: q_start[b] .. q_start[b+1]-1);
    ``max_q_len`` is the largest width."""

    def __init__(self, q, q_start, k_pages, v_pages, page_table, kv_lens, max_q_len, max_kv_len,
                 k_scales=None, v_scales=None, sm_scale=None, num_splits=0, with_lse=True, window=0, sink=0):
        dev = q.device
        B = kv_lens.shape[0]
        Hq, D = q.shape[1], q.shape[2]
        Hkv, P = k_pages.shape[1], k_pages.shape[2]
        dtype = SV_KV_FP8_E4M3 if k_pages.dtype == torch.uint8 else SV_KV_FP16
        self.params = make_params(B, max_q_len, Hq, Hkv, D, P, k_pages.shape[0], page_table.shape[1],
                                  max_kv_len, dtype, sm_scale, num_splits, window, sink)
        self.q_start = q_start
        self.inputs = (q, k_pages, v_pages, k_scales, v_scales, page_table, kv_lens)
        self.out = torch.empty_like(q)
        self.out_lse = torch.empty((q.shape[0], Hq), dtype=torch.float32, device=dev) if with_lse else None
        nbytes = sv_verify_workspace_bytes(self.params)
        # zero-filled once: its first 32 KB are work counters every call leaves at zero
        self.workspace = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
        self.flags = torch.zeros(1, dtype=torch.int32, device=dev)
        self.splits, self.chunk = sv_verify_plan(self.params)
        self.kernel = sv_verify_plan_kernel(self.params)

    def run(self, stream=None):
        sv_verify_attention_ragged(self.params, self.q_start, *self.inputs, self.out, self.out_lse, self.workspace,
                                   self.flags, stream)
        return self.out, self.out_lse


class RaggedAcceptCall:
    def __init__(self, logits, block_ids, q_start, batch, max_q_len, kv_lens=None, with_argmax=True):
        dev = logits.device
        self.batch, self.max_q_len, self.vocab = batch, max_q_len, logits.shape[1]
        self.logits, self.block_ids, self.q_start = logits, block_ids, q_start
        self.accept_len = torch.empty(batch, dtype=torch.int32, device=dev)
        self.bonus = torch.empty(batch, dtype=torch.int32, device=dev)
        self.argmax = torch.empty(logits.shape[0], dtype=torch.int32, device=dev) if with_argmax else None
        self.kv_in = kv_lens
        self.kv_out = torch.empty_like(kv_lens) if kv_lens is not None else None
        nbytes = sv_greedy_accept_workspace_bytes(batch, max_q_len, self.vocab)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        self.flags = torch.zeros(1, dtype=torch.int32, device=dev)

    def run(self, stream=None):
        sv_greedy_accept_ragged(self.logits, self.block_ids, self.q_start, self.batch, self.max_q_len, self.vocab,
                                self.accept_len, self.bonus, self.argmax, self.kv_in, self.kv_out, self.workspace,
                                self.flags, stream)
        return self.accept_len, self.bonus, self.argmax, self.kv_out


class PrepareCall:
    """Outputs of one block preparation: q_start [B+1], positions, cache
    slots and block ids (each [B*max_q_len], the first q_start[B] written)
    and the cache lengths the verify pass sees."""

    def __init__(self, seq_lens, q_lens, page_table, max_q_len, page_size, num_pages, last_tokens=None,
                 draft_ids=None):
        dev = seq_lens.device
        B = seq_lens.shape[0]
        self.args = (seq_lens, q_lens, page_table, B, max_q_len, page_size, num_pages)
        i32 = dict(dtype=torch.int32, device=dev)
        self.q_start = torch.empty(B + 1, **i32)
        self.positions = torch.empty(B * max_q_len, **i32)
        self.cache_slot = torch.empty(B * max_q_len, **i32)
        self.kv_lens_out = torch.empty(B, **i32)
        self.last_tokens, self.draft_ids = last_tokens, draft_ids
        self.block_ids = torch.empty(B * max_q_len, **i32) if last_tokens is not None else None
        self.flags = torch.zeros(1, **i32)

    def run(self, stream=None):
        sv_prepare_block(*self.args, self.q_start, self.cache_slot, self.positions, self.kv_lens_out,
                         self.last_tokens, self.draft_ids, self.block_ids, self.flags, stream)
        return self


class RejectionAcceptCall:
    """Buffers of one stochastic-acceptance call (rejection sampling); the
    uniforms are the caller's."""

    def __init__(self, logits, draft_ids, draft_probs, q_len, temperature, u_accept, u_final, kv_lens=None):
        dev = logits.device
        self.batch = logits.shape[0] // q_len
        self.q_len, self.vocab, self.temperature = q_len, logits.shape[1], temperature
        self.inputs = (logits, draft_ids, draft_probs)
        self.u_accept, self.u_final = u_accept, u_final
        self.accept_len = torch.empty(self.batch, dtype=torch.int32, device=dev)
        self.token = torch.empty(self.batch, dtype=torch.int32, device=dev)
        self.kv_in = kv_lens
        self.kv_out = torch.empty_like(kv_lens) if kv_lens is not None else None
        nbytes = sv_rejection_accept_workspace_bytes(self.batch, q_len, self.vocab)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)

    def run(self, stream=None):
        lg, ids, dp = self.inputs
        sv_rejection_accept(lg, ids, dp, self.batch, self.q_len, self.vocab, self.temperature, self.u_accept,
                            self.u_final, self.accept_len, self.token, self.kv_in, self.kv_out, self.workspace, stream)
        return self.accept_len, self.token, self.kv_out


class TopkCall:
    """Buffers of one top-k candidate call over logits [rows, vocab]."""

    def __init__(self, logits, k=16):
        dev = logits.device
        rows, vocab = logits.shape
        self.logits, self.k = logits, k
        self.ids = torch.empty((rows, k), dtype=torch.int32, device=dev)
        self.values = torch.empty((rows, k), dtype=torch.float32, device=dev)
        nbytes = sv_topk_candidates_workspace_bytes(rows, vocab, k)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)

    def run(self, stream=None):
        sv_topk_candidates(self.logits, self.k, self.ids, self.values, self.workspace, stream)
        return self.ids, self.values
