"""The C ABI library loads, exports every entry point include/sv.h declares,
and rejects bad arguments on the host without launching (no GPU needed)."""
import ctypes
import os
import re

import pytest

from long_context_gqa_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "sv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_symbols()
    for n in ("sv_verify_attention", "sv_verify_merge", "sv_greedy_accept"):
        assert n in names
    assert set(names) == set(B.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    for n in declared_symbols():
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_status_strings_and_version():
    lib = B.lib()
    assert lib.sv_status_string(0) == b"SV_OK"
    assert lib.sv_status_string(3) == b"SV_ERR_WORKSPACE_TOO_SMALL"
    assert B.sv_version() >= 100


def _p(**kw):
    base = dict(batch=1, q_len=8, num_q_heads=24, num_kv_heads=4, head_dim=256, page_size=16,
                num_pages=300, max_pages_per_req=257, max_kv_len=4104)
    base.update(kw)
    return B.make_params(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(q_len=0), B.SV_ERR_UNSUPPORTED),
    (dict(q_len=513, max_kv_len=4104), B.SV_ERR_UNSUPPORTED),
    (dict(head_dim=128), B.SV_ERR_UNSUPPORTED),
    (dict(num_q_heads=25), B.SV_ERR_INVALID_ARGUMENT),
    (dict(page_size=24), B.SV_ERR_UNSUPPORTED),
    (dict(max_kv_len=7), B.SV_ERR_INVALID_ARGUMENT),
    (dict(max_kv_len=5000), B.SV_ERR_INVALID_ARGUMENT),  # beyond max_pages_per_req * page_size
    (dict(num_q_heads=64, num_kv_heads=2, q_len=257), B.SV_ERR_UNSUPPORTED),  # 8224 rows per KV head
    (dict(batch=0), B.SV_ERR_INVALID_ARGUMENT),
    (dict(num_pages=1 << 27), B.SV_ERR_UNSUPPORTED),  # 2^33 cache rows: beyond 32-bit row indices
])
def test_plan_rejects_bad_shapes(kw, status):
    with pytest.raises(B.SvError) as e:
        B.sv_verify_plan(_p(**kw))
    assert e.value.status == status
    assert B.sv_verify_workspace_bytes(_p(**kw)) == 0


def test_plan_accepts_extend_chunks_up_to_the_limits():
    # an extend chunk of 512 rows, and 8192 rows on one KV head (the maxima)
    for kw in (dict(q_len=512), dict(q_len=512, num_q_heads=16, num_kv_heads=1), dict(q_len=100)):
        p = _p(**kw)
        s, c = B.sv_verify_plan(p)
        assert s >= 1 and c % 64 == 0
        rows = p.batch * p.q_len * p.num_q_heads
        assert B.sv_verify_workspace_bytes(p) >= (0 if s == 1 else s * rows * 256 * 4)


def test_plan_chunks_are_anchored_multiples_of_64():
    for maxkv in (8, 100, 4104, 32776, 524296):
        p = _p(max_kv_len=maxkv, max_pages_per_req=(maxkv + 15) // 16, num_pages=(maxkv + 15) // 16)
        s, c = B.sv_verify_plan(p)
        assert c % 64 == 0 and s == -(-maxkv // c)
        assert (B.sv_verify_workspace_bytes(p) == 0) == (s == 1)
    for forced in (1, 2, 3, 7, 64):
        p = _p(num_splits=forced)
        s, c = B.sv_verify_plan(p)
        assert s <= forced and s == -(-4104 // c)


def test_null_pointers_rejected_without_launch():
    lib = B.lib()
    p = _p()
    st = lib.sv_verify_attention(ctypes.byref(p), None, None, None, None, None, None, None, None, None,
                                 None, 0, None, None)
    assert st == B.SV_ERR_INVALID_ARGUMENT
    assert b"non-NULL" in lib.sv_last_error()
    st = lib.sv_verify_merge(None, None, 1, 1, 1, 256, None, None, None)
    assert st == B.SV_ERR_INVALID_ARGUMENT
    st = lib.sv_greedy_accept(None, None, 1, 8, 100, None, None, None, None, None, None, 0, None)
    assert st == B.SV_ERR_INVALID_ARGUMENT


def test_workspace_too_small_rejected_without_launch():
    lib = B.lib()
    p = _p(num_splits=4)
    fake = 1 << 40  # never dereferenced: the call must fail before any launch
    st = lib.sv_verify_attention(ctypes.byref(p), fake, fake, fake, None, None, fake, fake, fake, None,
                                 fake, 16, None, None)
    assert st == B.SV_ERR_WORKSPACE_TOO_SMALL
    need = lib.sv_greedy_accept_workspace_bytes(2, 8, 248320)
    assert need == ((2 * 8 * 31 * 8 + 255) // 256) * 256
    st = lib.sv_greedy_accept(fake, fake, 2, 8, 248320, fake, fake, None, None, None, fake, need - 1, None)
    assert st == B.SV_ERR_WORKSPACE_TOO_SMALL
    st = lib.sv_greedy_accept(fake, fake, 2, 8, 248320, fake, fake, None, fake, None, fake, need, None)
    assert st == B.SV_ERR_INVALID_ARGUMENT  # kv_lens_in without kv_lens_out


def test_fp16_with_scales_rejected():
    lib = B.lib()
    p = _p()
    fake = 1 << 40
    st = lib.sv_verify_attention(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, None,
                                 fake, 1 << 30, None, None)
    assert st == B.SV_ERR_INVALID_ARGUMENT


def test_block_entry_points_reject_bad_arguments_without_launch():
    lib = B.lib()
    fake = 1 << 40
    p = _p(num_splits=4)
    # ragged attention: q_start is required, and the uniform checks still apply
    st = lib.sv_verify_attention_ragged(ctypes.byref(p), None, fake, fake, fake, None, None, fake, fake, fake,
                                        None, fake, 1 << 30, None, None)
    assert st == B.SV_ERR_INVALID_ARGUMENT and b"q_start" in lib.sv_last_error()
    st = lib.sv_verify_attention_ragged(ctypes.byref(p), fake, fake, fake, fake, None, None, fake, fake, fake,
                                        None, fake, 16, None, None)
    assert st == B.SV_ERR_WORKSPACE_TOO_SMALL
    st = lib.sv_verify_attention_ragged(ctypes.byref(_p(q_len=513)), fake, fake, fake, fake, None, None, fake,
                                        fake, fake, None, fake, 1 << 30, None, None)
    assert st == B.SV_ERR_UNSUPPORTED
    # ragged accept: q_start and (for widths > 1) block_ids are required
    need = lib.sv_greedy_accept_workspace_bytes(2, 8, 1000)
    st = lib.sv_greedy_accept_ragged(fake, fake, None, 2, 8, 1000, fake, fake, None, None, None, fake, need,
                                     None, None)
    assert st == B.SV_ERR_INVALID_ARGUMENT
    st = lib.sv_greedy_accept_ragged(fake, None, fake, 2, 8, 1000, fake, fake, None, None, None, fake, need,
                                     None, None)
    assert st == B.SV_ERR_INVALID_ARGUMENT and b"block_ids" in lib.sv_last_error()
    st = lib.sv_greedy_accept_ragged(fake, fake, fake, 2, 8, 1000, fake, fake, None, None, None, fake, need - 1,
                                     None, None)
    assert st == B.SV_ERR_WORKSPACE_TOO_SMALL
    # prepare_block
    st = lib.sv_prepare_block(fake, fake, fake, 0, 8, 4, 16, 100, None, None, fake, None, fake, None, None,
                              None, None)
    assert st == B.SV_ERR_INVALID_ARGUMENT
    st = lib.sv_prepare_block(fake, fake, fake, 2, 8, 4, 16, 1 << 28, None, None, fake, None, fake, None, None,
                              None, None)
    assert st == B.SV_ERR_UNSUPPORTED  # flat slots past int32
    st = lib.sv_prepare_block(fake, fake, fake, 2, 8, 4, 16, 100, fake, None, fake, None, fake, None, None,
                              None, None)
    assert st == B.SV_ERR_INVALID_ARGUMENT  # last_tokens without block_ids
    st = lib.sv_prepare_block(fake, fake, fake, 2, 8, 4, 16, 100, fake, None, fake, None, fake, None, fake,
                              None, None)
    assert st == B.SV_ERR_INVALID_ARGUMENT and b"draft_ids" in lib.sv_last_error()
    # append_kv
    st = lib.sv_append_kv(fake, fake, fake, fake, 2, 16, 4, 256, 16, 100, B.SV_KV_FP8_E4M3, fake, fake, None,
                          None)
    assert st == B.SV_ERR_UNSUPPORTED
    st = lib.sv_append_kv(fake, fake, fake, fake, 2, 16, 4, 250, 16, 100, B.SV_KV_FP16, fake, fake, None, None)
    assert st == B.SV_ERR_UNSUPPORTED  # head_dim not a multiple of 8
    st = lib.sv_append_kv(fake + 8, fake, fake, fake, 2, 16, 4, 256, 16, 100, B.SV_KV_FP16, fake, fake, None,
                          None)
    assert st == B.SV_ERR_INVALID_ARGUMENT  # misaligned
    st = lib.sv_append_kv(None, fake, fake, fake, 2, 16, 4, 256, 16, 100, B.SV_KV_FP16, fake, fake, None, None)
    assert st == B.SV_ERR_INVALID_ARGUMENT
    # append_kv_fp8: head_dim a multiple of 64, scale pages required, alignment
    st = lib.sv_append_kv_fp8(fake, fake, fake, fake, 2, 16, 4, 96, 16, 100, fake, fake, fake, fake, None, None)
    assert st == B.SV_ERR_UNSUPPORTED
    st = lib.sv_append_kv_fp8(fake, fake, fake, fake, 2, 16, 4, 256, 16, 100, fake, fake, None, fake, None, None)
    assert st == B.SV_ERR_INVALID_ARGUMENT and b"k_scales" in lib.sv_last_error()
    st = lib.sv_append_kv_fp8(fake + 4, fake, fake, fake, 2, 16, 4, 256, 16, 100, fake, fake, fake, fake, None,
                              None)
    assert st == B.SV_ERR_INVALID_ARGUMENT  # new_k not 8-byte aligned
    st = lib.sv_append_kv_fp8(fake, fake, fake, fake, 0, 16, 4, 256, 16, 100, fake, fake, fake, fake, None, None)
    assert st == B.SV_ERR_INVALID_ARGUMENT


def test_rejection_accept_rejects_bad_arguments_without_launch():
    lib = B.lib()
    fake = 1 << 40
    need = lib.sv_rejection_accept_workspace_bytes(4, 8, 248320)
    assert need == 4 * 8 * 31 * 8 + ((4 * 31 * 4 + 255) // 256) * 256 + 256
    ok = [fake, fake, fake, 4, 8, 248320, 1.0, fake, fake, fake, fake, None, None, fake, need, None]

    def call(**kw):
        args = list(ok)
        names = ["logits", "ids", "probs", "batch", "q", "vocab", "T", "ua", "uf", "acc", "tok", "kin", "kout",
                 "ws", "wsb", "stream"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return lib.sv_rejection_accept(*args)

    assert call(T=0.0) == B.SV_ERR_INVALID_ARGUMENT
    assert call(T=float("nan")) == B.SV_ERR_INVALID_ARGUMENT
    assert call(q=65) == B.SV_ERR_UNSUPPORTED
    assert call(probs=None) == B.SV_ERR_INVALID_ARGUMENT
    assert call(kin=fake) == B.SV_ERR_INVALID_ARGUMENT
    assert call(wsb=need - 1) == B.SV_ERR_WORKSPACE_TOO_SMALL
    assert call(logits=fake + 4) == B.SV_ERR_INVALID_ARGUMENT


def test_topk_rejects_bad_arguments_without_launch():
    lib = B.lib()
    fake = 1 << 40
    need = lib.sv_topk_candidates_workspace_bytes(8, 248320, 16)
    assert need == 8 * 31 * 16 * 8  # a list of 16 (value, index) pairs per (row, 8,192-column slice)
    assert lib.sv_topk_candidates(fake, 8, 248320, 17, fake, fake, fake, need, None) == B.SV_ERR_UNSUPPORTED
    assert lib.sv_topk_candidates(fake, 8, 248320, 0, fake, fake, fake, need, None) == B.SV_ERR_UNSUPPORTED
    assert lib.sv_topk_candidates(fake, 8, 10, 11, fake, fake, fake, need, None) == B.SV_ERR_INVALID_ARGUMENT
    assert lib.sv_topk_candidates(fake, 8, 1 << 20, 16, fake, fake, fake, 1 << 30, None) == B.SV_ERR_UNSUPPORTED
    assert lib.sv_topk_candidates(fake, 8, 248320, 16, fake, fake, fake, need - 1, None) == B.SV_ERR_WORKSPACE_TOO_SMALL
    assert lib.sv_topk_candidates(None, 8, 248320, 16, fake, fake, fake, need, None) == B.SV_ERR_INVALID_ARGUMENT


def test_window_parameters_are_validated():
    with pytest.raises(B.SvError) as e:
        B.sv_verify_plan(_p(window=-1))
    assert e.value.status == B.SV_ERR_INVALID_ARGUMENT
    with pytest.raises(B.SvError) as e:
        B.sv_verify_plan(_p(sink=4))  # a sink without a window
    assert e.value.status == B.SV_ERR_INVALID_ARGUMENT
    assert B.sv_verify_plan(_p(window=2048, sink=4))[0] >= 1


def test_options_are_validated_and_claimed_work_needs_a_flag_word():
    # unknown option bits are refused on the host
    with pytest.raises(B.SvError) as e:
        B.sv_verify_plan(_p(options=0x2))
    assert e.value.status == B.SV_ERR_INVALID_ARGUMENT
    # one 512K request: the default plan and the claimed-work option both
    # plan 64 splits; with the option the call needs a status_flags word
    # (a dirty counter block is reported only there) and is refused first
    kw = dict(max_kv_len=524296, max_pages_per_req=32769, num_pages=32769)
    assert B.sv_verify_plan(_p(**kw)) == B.sv_verify_plan(_p(options=B.SV_VERIFY_CLAIMED_WORK, **kw))
    lib = B.lib()
    fake = 1 << 40
    p = _p(options=B.SV_VERIFY_CLAIMED_WORK, **kw)
    need = B.sv_verify_workspace_bytes(p)
    st = lib.sv_verify_attention(ctypes.byref(p), fake, fake, fake, None, None, fake, fake, fake, None,
                                 fake, need, None, None)
    assert st == B.SV_ERR_INVALID_ARGUMENT and b"status_flags" in lib.sv_last_error()


def test_noalloc_entry_point_refuses_plans_beyond_its_scratch():
    # the ragged 32 x 131K q=16 workload's plan needs about 200 MB of
    # workspace: more than the library's 32 MiB scratch, refused before any
    # device call
    lib = B.lib()
    assert B.sv_verify_scratch_bytes() == 32 << 20
    p = _p(batch=32, q_len=16, page_size=64, max_kv_len=131088, max_pages_per_req=2049, num_pages=65568)
    assert B.sv_verify_workspace_bytes(p) > B.sv_verify_scratch_bytes()
    fake = 1 << 40
    st = lib.sv_verify_attention_noalloc(ctypes.byref(p), fake, fake, fake, None, None, fake, fake, fake, None,
                                         None, None)
    assert st == B.SV_ERR_WORKSPACE_TOO_SMALL and b"scratch" in lib.sv_last_error()
    # bad shapes are refused as by sv_verify_attention
    st = lib.sv_verify_attention_noalloc(ctypes.byref(_p(head_dim=128)), fake, fake, fake, None, None, fake, fake,
                                         fake, None, None, None)
    assert st == B.SV_ERR_UNSUPPORTED


@pytest.mark.parametrize("batch,q_len,max_kv,page,dtype,splits", [
    (1, 8, 4104, 16, B.SV_KV_FP16, 33),            # 4K: chunks of 128 (the smallest)
    (8, 8, 32776, 16, B.SV_KV_FP16, 8),            # 8 x 32K: one round, XCD-balanced
    (1, 8, 524296, 16, B.SV_KV_FP16, 64),          # 512K: one workgroup per CU, XCD-balanced
    (32, 16, 131088, 64, B.SV_KV_FP16, 16),        # ragged q=16 bound: the two-half kernel's 8K-token cap
    (4, 8, 262152, 16, B.SV_KV_FP8_E4M3, 16),      # FP8 4 x 262K: one workgroup per CU (under its 32K cap)
])
def test_plans_of_the_benchmark_workloads(batch, q_len, max_kv, page, dtype, splits):
    # the planner's choices for the five workloads (256 compute units assumed
    # when no GPU is present, as on the MI355X)
    pages = -(-max_kv // page)
    p = _p(batch=batch, q_len=q_len, page_size=page, max_kv_len=max_kv, max_pages_per_req=pages,
           num_pages=pages * batch, kv_dtype=dtype)
    s, c = B.sv_verify_plan(p)
    assert s == splits, (s, c)
    assert c % 64 == 0 and s * c >= max_kv


@pytest.mark.parametrize("batch,q_len,max_kv,page,dtype,splits,kernel", [
    # 96 rows per KV head, fp16, automatic splits: the two-half kernel only
    # where its chunks are at least 2,048 positions long
    (1, 16, 13000, 16, B.SV_KV_FP16, 0, B.SV_KERNEL_ROW_TILES),     # 53 MB, chunks of 256 for the halves
    (1, 16, 65000, 16, B.SV_KV_FP16, 0, B.SV_KERNEL_ROW_TILES),     # chunks of 1,024 for the halves
    (4, 16, 16500, 16, B.SV_KV_FP16, 0, B.SV_KERNEL_ROW_TILES),     # chunks of 1,088 for the halves
    (1, 16, 131000, 16, B.SV_KV_FP16, 0, B.SV_KERNEL_TWO_HALVES),   # chunks of 2,048
    (8, 16, 32776, 16, B.SV_KV_FP16, 0, B.SV_KERNEL_TWO_HALVES),
    (32, 16, 131088, 64, B.SV_KV_FP16, 0, B.SV_KERNEL_TWO_HALVES),  # the ragged batch's bound: 8K-token chunks
    (1, 16, 524296, 16, B.SV_KV_FP16, 0, B.SV_KERNEL_TWO_HALVES),
    # forced splits keep it down to the shortest chunks (tests of the pipeline's edge rounds)
    (2, 16, 4200, 16, B.SV_KV_FP16, 33, B.SV_KERNEL_TWO_HALVES),
    (1, 16, 13000, 16, B.SV_KV_FP16, 5, B.SV_KERNEL_TWO_HALVES),
    # under 32 MB, at most 48 rows, FP8 keys, or chunks beyond 32,768: row tiles
    (2, 16, 3000, 16, B.SV_KV_FP16, 33, B.SV_KERNEL_ROW_TILES),
    (1, 8, 524296, 16, B.SV_KV_FP16, 0, B.SV_KERNEL_ROW_TILES),
    (1, 16, 524296, 16, B.SV_KV_FP8_E4M3, 0, B.SV_KERNEL_ROW_TILES),
    (1, 16, 131000, 16, B.SV_KV_FP16, 2, B.SV_KERNEL_ROW_TILES),
])
def test_plan_kernel_choice(batch, q_len, max_kv, page, dtype, splits, kernel):
    pages = -(-max_kv // page)
    p = _p(batch=batch, q_len=q_len, page_size=page, max_kv_len=max_kv, max_pages_per_req=pages,
           num_pages=pages * batch, kv_dtype=dtype, num_splits=splits)
    assert B.sv_verify_plan_kernel(p) == kernel
    if kernel == B.SV_KERNEL_TWO_HALVES:
        s, c = B.sv_verify_plan(p)
        assert c <= 32768 and (splits > 0 or c >= 2048), (s, c)


def test_plan_kernel_rejects_null_and_bad_shapes():
    lib = B.lib()
    assert lib.sv_verify_plan_kernel(ctypes.byref(_p()), None) == B.SV_ERR_INVALID_ARGUMENT
    k = ctypes.c_int32(-1)
    assert lib.sv_verify_plan_kernel(ctypes.byref(_p(head_dim=128)), ctypes.byref(k)) == B.SV_ERR_UNSUPPORTED
    assert k.value == -1
