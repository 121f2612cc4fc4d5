"""GPU parity of claimed work (the SV_VERIFY_CLAIMED_WORK option) against the
float64 oracle: requests with fp16 keys whose split workgroups claim the keys
in grains at run time (split
count a multiple of 8, at least 64 key steps per wave). Covered: forced 8
and 16 splits over a 40K cache (static first segments, then grains, a last
grain that ends inside a page), the same plan over much shorter actual
lengths (no static segment, a handful of grains for many waves, empty
workgroups), one and two row blocks, agreement with the static split of the
same call, repeated calls, and the work counters in the workspace's first
32 KB (left zero by every call; a call on a workspace whose counters are not
zero raises bit 0x10)."""
import numpy as np
import pytest
import torch

from helpers import case, check, host, oracle, rows_of, run_gpu, say
from long_context_gqa_amd import binding as B

pytestmark = pytest.mark.gpu

KV = 40003  # >= 4096 * 8: claimed work with 8 splits; not a multiple of 16


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def plan(x, splits, max_kv, claim=True):
    c = B.VerifyCall(x.q, x.k_pages, x.v_pages, x.page_table.cuda().contiguous(), x.kv_lens.cuda(), x.wl.q_len,
                     max_kv, x.k_scales, x.v_scales, x.sm_scale, splits, claim=claim)
    return c


@pytest.mark.parametrize("q_len,splits,variant", [(8, 8, "unit"), (8, 16, "literal"), (4, 8, "unit"),
                                                  (1, 8, "unit")])
def test_claimed_work_matches_oracle(q_len, splits, variant):
    x = case(1, q_len, [KV], 16, variant, seed=40 + q_len + splits)
    c = plan(x, splits, KV)
    say(f"q={q_len} splits={splits} {variant}: plan {c.splits} x {c.chunk}")
    assert c.splits == splits
    out, lse, flags = run_gpu(x, num_splits=splits, claim=True)
    assert flags == 0
    ref, ref_lse = oracle(x)
    check(out, lse, ref, ref_lse, what=f"claimed q={q_len} S={splits}")
    # the static split of the same call (7 splits: not a multiple of 8)
    out7, lse7, flags7 = run_gpu(x, num_splits=7)
    assert flags7 == 0
    check(out7, lse7, ref, ref_lse, what="static S=7")
    assert np.abs(out - out7).max() <= 2e-3


# 2720 / 2736 / 2737: 170 / 171 / 172 steps, where a wave's static segment
# goes from none (all 170 steps claimed) to 4 steps, the last one partial
@pytest.mark.parametrize("kv", [8, 9, 300, 1000, 2720, 2736, 2737, 4097, 20000])
def test_claimed_work_over_shorter_actual_lengths(kv):
    # the plan (8 splits, 40K) asks for claimed work; the request is shorter:
    # below 4 * 32 * 4 = 512 steps there is no static segment, and only a few
    # of the 32 waves per KV head get a grain
    x = case(1, 8, [KV], 16, "unit", seed=9)
    kvl = torch.tensor([kv], dtype=torch.int32)
    out, lse, flags = run_gpu(x, num_splits=8, max_kv_len=KV, kv_lens=kvl, claim=True)
    assert flags == 0
    h = host(x)
    h["kv_lens"] = kvl
    ref, ref_lse = oracle(x, h=h)
    say(f"kv={kv}: max |err| {np.abs(out - ref).max():.2e}")
    check(out, lse, ref, ref_lse, what=f"kv={kv}")


def test_counters_left_zero_and_a_dirty_workspace_is_flagged():
    x = case(1, 8, [KV], 16, "unit", seed=12)
    c = plan(x, 8, KV)
    ref, ref_lse = oracle(x, groups=[(0, 2)])
    mask = rows_of(x, [(0, 2)])
    outs = []
    for i in range(3):
        c.flags.zero_()
        c.run()
        torch.cuda.synchronize()
        assert int(c.flags.item()) == 0
        assert int(c.workspace[:32768].count_nonzero().item()) == 0
        out = c.out.float().cpu().numpy()
        check(out, c.out_lse.cpu().numpy(), ref, ref_lse, mask=mask, what=f"call {i}")
        outs.append(out)
    # repeated calls agree to rounding (the grains' order varies)
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2e-3
    # a workspace whose counters are not zero: flagged, and cleared again.
    # Small, large (a leftover 1.0f, INT32_MAX) and negative values: a wave
    # takes a ticket only below its counter's grain count, so none of them
    # forms a grain index outside the cache
    # A counter a little above zero skips its first grains yet ends at the
    # clean value: the group's tally of grains taken (word 1) shows it; a
    # dirty tally alone is caught too
    ctr = c.workspace[:32768].view(torch.int32)
    cases = [(0, v) for v in (1, 3, 0x03030303, 0x3F800000, 0x7FFFFFFF, -5, -(1 << 31))] + [(1, 3), (1, -1)]
    for word, dirty in cases:
        ctr[word] = dirty
        if word == 0:
            ctr[5 * 64] = dirty  # the counter on the sixth 256-byte line
        c.flags.zero_()
        c.run()
        torch.cuda.synchronize()
        say(f"  dirty word {word} = {dirty}: flags {int(c.flags.item())}")
        assert int(c.flags.item()) & 0x10
        assert int(c.workspace[:32768].count_nonzero().item()) == 0
        assert torch.isfinite(c.out.float()).all()
        c.flags.zero_()
        c.run()
        torch.cuda.synchronize()
        assert int(c.flags.item()) == 0
        check(c.out.float().cpu().numpy(), c.out_lse.cpu().numpy(), ref, ref_lse, mask=mask,
              what=f"after the reset (word {word} = {dirty})")


@pytest.mark.parametrize("lens,splits", [([KV] * 3, 8), ([KV, 9000, 300, KV - 20, 17], 8), ([70000, 70000], 16)])
def test_batches_keep_the_static_order(lens, splits):
    # several requests never claim (their lengths may be ragged), even with
    # the option: the same plans as above over batches take static chunks
    # (XCD-balanced ones where the grid fits the GPU in one round), are
    # exact against the oracle and give the same bits on every call
    x = case(len(lens), 8, lens, 16, "unit", seed=len(lens) + splits)
    c = plan(x, splits, max(lens))
    say(f"batch {len(lens)} lens {lens} splits {splits}: plan {c.splits} x {c.chunk}")
    out, lse, flags = run_gpu(x, num_splits=splits, claim=True)
    assert flags == 0
    c.run()
    torch.cuda.synchronize()
    first = c.out.clone()
    c.run()
    torch.cuda.synchronize()
    assert torch.equal(first, c.out)
    groups = [(b, g) for b in range(len(lens)) for g in (0, 3)]
    ref, ref_lse = oracle(x, groups=groups)
    check(out, lse, ref, ref_lse, mask=rows_of(x, groups), what=f"batch {len(lens)}")



@pytest.mark.parametrize("page,q_len,Hq,Hkv", [(64, 8, 24, 4), (48, 8, 24, 4), (16, 16, 24, 8), (32, 4, 16, 8)])
def test_claimed_work_pages_and_heads(page, q_len, Hq, Hkv):
    # steps of 16 positions inside larger pages (48: not a power of two), and
    # 8 KV heads (three or two query heads each; 48 or 8 rows per KV head)
    x = case(1, q_len, [KV], page, "unit", seed=page + q_len + Hkv, Hq=Hq, Hkv=Hkv)
    c = plan(x, 8, KV)
    say(f"P={page} q={q_len} Hq={Hq} Hkv={Hkv}: plan {c.splits} x {c.chunk}")
    out, lse, flags = run_gpu(x, num_splits=8, claim=True)
    assert flags == 0
    groups = [(0, 0), (0, Hkv - 1)]
    ref, ref_lse = oracle(x, groups=groups)
    check(out, lse, ref, ref_lse, mask=rows_of(x, groups), what=f"P={page} Hkv={Hkv}")


def test_claimed_work_replays_in_a_graph():
    # the counters must be back at zero after every replay (the merge clears
    # them with plain stores inside the graph); each replay, with an eager
    # call between, is checked against the oracle and must raise no flag
    x = case(1, 8, [KV], 16, "unit", seed=21)
    c = plan(x, 8, KV)
    ref, ref_lse = oracle(x, groups=[(0, 1)])
    mask = rows_of(x, [(0, 1)])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            c.flags.zero_()
            c.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c.flags.zero_()
        c.run()
    torch.cuda.synchronize()
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert int(c.flags.item()) == 0
        assert int(c.workspace[:32768].count_nonzero().item()) == 0
        check(c.out.float().cpu().numpy(), c.out_lse.cpu().numpy(), ref, ref_lse, mask=mask, what=f"replay {r}")
        out2, lse2, flags2 = run_gpu(x, num_splits=8, claim=True)  # eager work between replays
        assert flags2 == 0
