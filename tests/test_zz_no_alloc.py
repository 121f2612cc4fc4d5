"""The allocation-free verify entry point (sv_verify_attention_noalloc: the
workspace in the library's own device scratch) against sv_verify_attention
with a caller workspace, through the C ABI: the same plan and kernels, so the
same bits, on calls in a row over shrinking inputs (the 512K single request,
a 131K request at q = 16 on the two-half kernel, a 40K request on 8
XCD-balanced splits, a 12K request at q = 16 on the two-half kernel with
forced splits, a batch of two 6K requests), and the
claimed-work option, whose counters live at the start of the scratch (zero
at load, left zero by every call)."""
import numpy as np
import pytest
import torch

from helpers import case, check, oracle, rows_of, say
from long_context_gqa_amd import binding as B
from long_context_gqa_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def both(x, splits=0, claim=False, max_kv=None):
    """(workspace call's out, lse, flags), (no-alloc call's out, lse, flags)"""
    mk = max_kv if max_kv is not None else int(x.kv_lens.max())
    c = B.VerifyCall(x.q, x.k_pages, x.v_pages, x.page_table.cuda().contiguous(), x.kv_lens.cuda(), x.wl.q_len,
                     mk, x.k_scales, x.v_scales, x.sm_scale, splits, claim=claim)
    c.run()
    out = torch.empty_like(x.q)
    lse = torch.empty((x.q.shape[0], x.q.shape[1]), dtype=torch.float32, device="cuda")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.sv_verify_attention_noalloc(c.params, x.q, x.k_pages, x.v_pages, x.k_scales, x.v_scales, c.inputs[5],
                                  c.inputs[6], out, lse, flags)
    torch.cuda.synchronize()
    say(f"  plan {c.splits} x {c.chunk}, workspace {B.sv_verify_workspace_bytes(c.params)} bytes")
    return (c.out, c.out_lse, int(c.flags.item())), (out, lse, int(flags.item()))


def test_noalloc_matches_the_workspace_call_on_shrinking_inputs():
    # (the 131K and 12K blocks of 96 rows per KV head run on the two-half kernel)
    cases = [("512K", lambda: W.make_verify_inputs(W.WORKLOADS[3], "unit", device="cuda"), 0, None),
             ("131K at q=16", lambda: case(1, 16, [131000], 16, "unit", seed=8), 0, B.SV_KERNEL_TWO_HALVES),
             ("40K, 8 splits", lambda: case(1, 8, [40003], 16, "unit", seed=5), 8, None),
             ("12K at q=16, 5 splits", lambda: case(1, 16, [12001], 16, "unit", seed=9), 5, B.SV_KERNEL_TWO_HALVES),
             ("2 x 6K", lambda: case(2, 8, [6000, 5100], 16, "unit", seed=6), 0, None)]
    for name, make, splits, kernel in cases:
        x = make()
        if kernel is not None:
            c = B.VerifyCall(x.q, x.k_pages, x.v_pages, x.page_table.cuda(), x.kv_lens.cuda(), x.wl.q_len,
                             int(x.kv_lens.max()), None, None, x.sm_scale, splits)
            assert c.kernel == kernel
            del c
        (o1, l1, f1), (o2, l2, f2) = both(x, splits)
        say(f"{name}: bitwise equal {torch.equal(o1, o2) and torch.equal(l1, l2)}")
        assert f1 == 0 and f2 == 0
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        del x
        torch.cuda.empty_cache()


def test_noalloc_with_claimed_work_counters_in_the_scratch():
    # the counters at the scratch's start were zero at load and every call
    # leaves them zero: two claimed calls in a row raise no flag and match
    # the oracle; the second over a shorter actual length
    x = case(1, 8, [40003], 16, "unit", seed=7)
    ref, ref_lse = oracle(x, groups=[(0, 1)])
    mask = rows_of(x, [(0, 1)])
    for kv in (40003, 9000):
        if kv != 40003:
            x.kv_lens = torch.tensor([kv], dtype=torch.int32)
            ref, ref_lse = oracle(x, groups=[(0, 1)])
        # the plan of a 40K bound in both calls (claimed work: 8 splits)
        (o1, l1, f1), (o2, l2, f2) = both(x, 8, claim=True, max_kv=40003)
        assert f1 == 0 and f2 == 0
        check(o2.float().cpu().numpy(), l2.cpu().numpy(), ref, ref_lse, mask=mask, what=f"no-alloc claimed kv={kv}")
        assert (o1.float() - o2.float()).abs().max().item() <= 2e-3
