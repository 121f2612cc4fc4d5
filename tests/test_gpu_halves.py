"""GPU parity of the two-half verify kernel (verify_rows.hip) against the
float64 oracle. The planner takes that kernel for 49 to 96 rows per KV head
with fp16 keys over a pass of 32 MB or more (each case here is sized above
that) when its chunks are at least 2,048 positions long, or for any chunk up
to 32,768 positions when the split count is forced: blocks of q = 9..16 at 6
query heads per KV head (54..96 rows, halves of 32 or 48 rows) and q = 8, 12
at 8, forced split counts (chunks of odd and even step counts, and chunks of
2 to 8 steps, where only the pipeline's first and last rounds run) and the
planner's own choice over long passes, pages of 16 to 64 positions, a
sliding window, blocks of a width per request, a request whose rows see no
key, and repeated and page-permuted calls that must give the same bits.
Each call first asks the planner which kernel it launches."""
import numpy as np
import pytest
import torch

from helpers import case, check, host, oracle, run_gpu, say
from long_context_gqa_amd import binding as B
from long_context_gqa_amd import workloads as W
from oracle import attention as oatt

pytestmark = pytest.mark.gpu

# the planner's threshold: B * Hkv * max_kv_len * 1 KB (fp16 K and V rows)
LARGE = 32 << 20


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def large(batch, Hkv, max_kv):
    return batch * Hkv * max_kv * 1024 >= LARGE


def plan_kernel(x, splits, max_kv=None, window=0, sink=0):
    """The kernel the plan launches for this call (SV_KERNEL_*)."""
    mk = max_kv if max_kv is not None else int(x.kv_lens.max())
    p = B.make_params(x.wl.batch, x.wl.q_len, x.q.shape[1], x.k_pages.shape[1], x.q.shape[2], x.k_pages.shape[2],
                      x.k_pages.shape[0], x.page_table.shape[1], mk, B.SV_KV_FP16, x.sm_scale, splits, window, sink)
    return B.sv_verify_plan_kernel(p)


def halves_expected(x, splits, max_kv=None):
    """Forced splits take the two-half kernel while the chunk fits its
    32,768-position cache-row table."""
    mk = max_kv if max_kv is not None else int(x.kv_lens.max())
    return -(-mk // splits) <= 32768


@pytest.mark.parametrize("B_,q,lens,P,Hq,Hkv,variant", [
    (2, 16, [4200, 4133], 16, 24, 4, "unit"),      # 96 rows: halves of 48
    (2, 16, [4200, 4133], 16, 24, 4, "literal"),
    (2, 9, [4500, 4100], 64, 24, 4, "unit"),       # 54 rows: halves of 32
    (3, 11, [3000, 2800, 5000], 32, 24, 4, "unit"),  # 66 rows: halves of 48, part empty
    (2, 8, [4300, 4096], 16, 32, 4, "unit"),       # G = 8: 64 rows
    (2, 12, [4300, 4111], 16, 32, 4, "unit"),      # G = 8: 96 rows
    (1, 16, [33000], 16, 24, 4, "unit"),           # one long request
])
def test_halves_parity(B_, q, lens, P, Hq, Hkv, variant):
    assert large(B_, Hkv, max(lens))
    x = case(B_, q, lens, P, variant, seed=q * 10 + B_, Hq=Hq, Hkv=Hkv)
    ref, ref_lse = oracle(x)
    # 1: one chunk (rows written directly); 3, 7: long chunks; 33, 66:
    # chunks of 8 and 4 steps (the pipeline's edge rounds)
    for splits in (1, 3, 7, 33, 66):
        kern = plan_kernel(x, splits)
        say(f"B={B_} q={q} lens={lens} P={P} Hq={Hq} Hkv={Hkv} {variant} splits={splits} kernel={kern}")
        assert kern == (B.SV_KERNEL_TWO_HALVES if halves_expected(x, splits) else B.SV_KERNEL_ROW_TILES)
        out, lse, flags = run_gpu(x, num_splits=splits)
        assert flags == 0
        check(out, lse, ref, ref_lse, what=f"splits={splits}")


@pytest.mark.parametrize("B_,q,lens,Hq", [
    (1, 16, [131000], 24),          # 96 rows, 64 chunks of 2,048
    (2, 12, [65536, 61000], 32),    # G = 8: 96 rows, 32 chunks of 2,048
])
def test_halves_planner_choice_on_long_passes(B_, q, lens, Hq):
    x = case(B_, q, lens, 16, "unit", seed=q * 7 + B_, Hq=Hq)
    assert plan_kernel(x, 0) == B.SV_KERNEL_TWO_HALVES
    ref, ref_lse = oracle(x)
    say(f"B={B_} q={q} lens={lens} Hq={Hq} planner's splits")
    out, lse, flags = run_gpu(x)
    assert flags == 0
    check(out, lse, ref, ref_lse, what="planner's splits")


def test_halves_window():
    B_, q, lens, Wn, S = 2, 16, [20000, 12000], 5000, 4
    assert large(B_, 4, S + Wn + q + 48)
    x = case(B_, q, lens, 16, "unit", seed=91)
    h = host(x)
    ref, ref_lse = oatt.verify_attention_window(h["q"], h["k_pages"], h["v_pages"], h["page_table"], h["kv_lens"],
                                                q, x.sm_scale, Wn, S, None, None)
    # 1, 5: the two-half kernel; 0: the planner's choice (row tiles: the
    # window's chunks are short)
    for splits in (1, 5, 0):
        kern = plan_kernel(x, splits, window=Wn, sink=S)
        say(f"window {Wn} sink {S} splits={splits} kernel={kern}")
        if splits:
            assert kern == B.SV_KERNEL_TWO_HALVES
        out, lse, flags = B.verify_attention(x.q, x.k_pages, x.v_pages, x.page_table.cuda(), x.kv_lens.cuda(), q,
                                             int(x.kv_lens.max()), None, None, x.sm_scale, splits, window=Wn,
                                             sink=S)
        torch.cuda.synchronize()
        assert int(flags.item()) == 0
        check(out.float().cpu().numpy(), lse.cpu().numpy(), ref, ref_lse, what=f"window splits={splits}")


def test_halves_widths_per_request():
    widths, prefixes, P = [16, 3, 9, 12, 1], [4000, 5000, 100, 4500, 3100], 16
    qmax = max(widths)
    assert large(len(widths), 4, max(p + w for p, w in zip(prefixes, widths)))
    wl = W.Workload("halves", len(widths), qmax, ("fixed", 0), P, seed=93)
    x = W.make_verify_inputs(wl, "unit", device="cuda", kv_lens=[L + qmax for L in prefixes])
    kv = torch.tensor([L + w for L, w in zip(prefixes, widths)], dtype=torch.int32)
    q = W.pack_rows(x.q, qmax, widths)
    qs = W.row_offsets(widths)
    h = host(x)
    ref, ref_lse = oatt.verify_attention_ragged(q.cpu(), h["k_pages"], h["v_pages"], h["page_table"], kv,
                                                np.array(widths), qs.numpy(), x.sm_scale, None, None)
    for splits in (1, 7, 0):
        c = B.RaggedVerifyCall(q, qs.cuda(), x.k_pages, x.v_pages, x.page_table.cuda(), kv.cuda(), qmax,
                               int(x.kv_lens.max()), None, None, x.sm_scale, splits)
        say(f"widths {widths} splits={splits} kernel={c.kernel}")
        if splits:
            assert c.kernel == B.SV_KERNEL_TWO_HALVES
        c.run()
        torch.cuda.synchronize()
        assert int(c.flags.item()) == 0
        check(c.out.float().cpu().numpy(), c.out_lse.cpu().numpy(), ref, ref_lse, what=f"splits={splits}")


def test_halves_repeat_and_page_permutation_bitwise():
    lens, splits = [4200, 4133], 7
    x = case(2, 16, lens, 16, "unit", seed=95)
    assert plan_kernel(x, splits) == B.SV_KERNEL_TWO_HALVES
    out, lse, _ = run_gpu(x, num_splits=splits)
    out_b, lse_b, _ = run_gpu(x, num_splits=splits)
    assert np.array_equal(out, out_b) and np.array_equal(lse, lse_b)
    n = x.k_pages.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(5))
    inv = torch.argsort(perm)
    x2 = case(2, 16, lens, 16, "unit", seed=95)
    x2.k_pages = x.k_pages[perm.cuda()].contiguous()
    x2.v_pages = x.v_pages[perm.cuda()].contiguous()
    t = x.page_table.clone()
    t[t >= 0] = inv[t[t >= 0].long()].to(torch.int32)
    x2.page_table = t
    out2, lse2, _ = run_gpu(x2, num_splits=splits)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_halves_request_with_rows_but_no_visible_key():
    # kv_len 0 for request 1 (below its block of 16): its rows get 0 and -inf
    # and the flag (its chunk has no step: only the pipeline's edge rounds
    # run); every other request matches the oracle
    lens, q = [4200, 900, 4133, 2500], 16
    assert large(len(lens), 4, max(lens))
    x = case(len(lens), q, lens, 16, "unit", seed=97)
    kv = x.kv_lens.clone()
    kv[1] = 0
    for splits in (1, 3, 0):
        kern = plan_kernel(x, splits)
        say(f"no visible key, splits={splits} kernel={kern}")
        if splits:
            assert kern == B.SV_KERNEL_TWO_HALVES
        out, lse, flags = run_gpu(x, num_splits=splits, kv_lens=kv, max_kv_len=max(lens))
        assert flags & 2
        assert (out[q:2 * q] == 0).all() and np.isneginf(lse[q:2 * q]).all()
        h = host(x)
        keep = [b for b in range(len(lens)) if b != 1]
        ref, ref_lse = oatt.verify_attention(h["q"], h["k_pages"], h["v_pages"], h["page_table"], h["kv_lens"], q,
                                             x.sm_scale, rows=[(b, g) for b in keep for g in range(4)])
        rows = np.concatenate([np.arange(b * q, (b + 1) * q) for b in keep])
        check(out[rows], lse[rows], ref[rows], ref_lse[rows], what=f"other requests, splits={splits}")
