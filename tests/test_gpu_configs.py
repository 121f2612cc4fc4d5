"""The full-size workloads (4K, 8 x 32K, 512K with biased keys, ragged
8K-131K DFlash blocks of 16, 4 x 262K FP8) through the launch configuration
the benchmark times, checked against the oracle on the whole output, in both
value variants: every (request, KV head) group of the uniform workloads, and
for the ragged batch two KV heads of every request per variant (heads b, b+2
in one variant and b+1, b+3 in the other, so the two variants together cover
every group). Repeated calls give the same bits, and so does a call over a
page-permuted copy of the pool. Plus the GPU merge fed oracle partials."""
import time

import numpy as np
import pytest
import torch

from helpers import check, host, oracle, rows_of, run_gpu, say
from long_context_gqa_amd import binding as B
from long_context_gqa_amd import workloads as W
from oracle import attention as oatt

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def groups_of(wl, variant):
    Hkv = wl.num_kv_heads
    if wl.batch * Hkv <= 64:
        return [(b, g) for b in range(wl.batch) for g in range(Hkv)]
    r = 0 if variant == "literal" else 1
    return [(b, (b + r + k) % Hkv) for b in range(wl.batch) for k in (0, 2)]


def call_of(x, splits=0):
    return B.VerifyCall(x.q, x.k_pages, x.v_pages, x.page_table.cuda().contiguous(), x.kv_lens.cuda(),
                        x.wl.q_len, x.max_kv_len, x.k_scales, x.v_scales, x.sm_scale, splits)


@pytest.mark.parametrize("variant", ["literal", "unit"])
@pytest.mark.parametrize("wl_id", [1, 2, 3, 4, 5])
def test_full_size_config(wl_id, variant):
    wl = W.WORKLOADS[wl_id]
    say(f"config {wl_id} {wl.name} {variant}: generating")
    x = W.make_verify_inputs(wl, variant, device="cuda")
    say(f"  pool {tuple(x.k_pages.shape)}, max kv {x.max_kv_len}")
    c = call_of(x)
    c.run()
    torch.cuda.synchronize()
    assert int(c.flags.item()) == 0
    first = c.out.clone()
    c.run()
    torch.cuda.synchronize()
    assert torch.equal(first, c.out), "repeated calls differ"
    out, lse = c.out.float().cpu().numpy(), c.out_lse.cpu().numpy()
    assert np.isfinite(out).all()
    groups = groups_of(wl, variant)
    t0 = time.time()
    ref, ref_lse = oracle(x, groups=groups)
    say(f"  oracle on {len(groups)} of {wl.batch * wl.num_kv_heads} groups in {time.time() - t0:.1f} s")
    check(out, lse, ref, ref_lse, mask=rows_of(x, groups), what=f"config {wl_id} {variant}")
    del x, c
    torch.cuda.empty_cache()


@pytest.mark.parametrize("wl_id", [3, 5])
def test_full_size_page_permutation_is_bitwise(wl_id):
    # the same cache with its physical pages moved (and the table rewritten
    # alike): the kernel sees the same keys in the same order, so the output
    # is the same to the bit
    wl = W.WORKLOADS[wl_id]
    x = W.make_verify_inputs(wl, "unit", device="cuda")
    c = call_of(x)
    c.run()
    torch.cuda.synchronize()
    base = c.out.clone()
    n = x.k_pages.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(77)).cuda()
    moved = []
    for t in (x.k_pages, x.v_pages, x.k_scales, x.v_scales):
        if t is None:
            moved.append(None)
            continue
        m = torch.empty_like(t)
        m[perm] = t
        moved.append(m)
    table = perm.to(torch.int32)[x.page_table.cuda().long()].contiguous()
    c2 = B.VerifyCall(x.q, moved[0], moved[1], table, x.kv_lens.cuda(), wl.q_len, x.max_kv_len, moved[2],
                      moved[3], x.sm_scale)
    c2.run()
    torch.cuda.synchronize()
    assert int(c2.flags.item()) == 0
    same = torch.equal(base, c2.out)
    say(f"config {wl_id}: page-permuted call bitwise equal: {same}")
    assert same


def test_512k_split_count_invariance():
    wl = W.WORKLOADS[3]
    x = W.make_verify_inputs(wl, "unit", device="cuda")
    ref, ref_lse = oracle(x)
    outs = []
    for splits in (0, 16, 97, 300):
        out, lse, _ = run_gpu(x, num_splits=splits)
        check(out, lse, ref, ref_lse, what=f"512K splits={splits}")
        outs.append(out)
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2e-3


def test_gpu_merge_of_oracle_partials():
    # oracle partials over an uneven partition, rounded to fp32, merged on
    # the GPU, against the oracle's unsplit attention
    x = W.make_verify_inputs(W.WORKLOADS[1].with_(batch=2), "unit", device="cpu", kv_lens=[900, 1300])
    h = host(x)
    q = x.wl.q_len
    ref, ref_lse = oatt.verify_attention(h["q"], h["k_pages"], h["v_pages"], h["page_table"], h["kv_lens"], q,
                                         x.sm_scale)
    cuts = [0, 100, 101, 640, 1100, 1300, 2000]
    parts = [oatt.attention_partial(h["q"], h["k_pages"], h["v_pages"], h["page_table"], h["kv_lens"], q,
                                    x.sm_scale, lo, hi) for lo, hi in zip(cuts[:-1], cuts[1:])]
    po = torch.tensor(np.stack([p[0] for p in parts]), dtype=torch.float32).cuda()
    pl = torch.tensor(np.stack([p[1] for p in parts]), dtype=torch.float32).cuda()
    out = torch.empty(po.shape[1:], dtype=torch.float16, device="cuda")
    lse = torch.empty(pl.shape[1:], dtype=torch.float32, device="cuda")
    B.sv_verify_merge(po, pl, out, lse)
    torch.cuda.synchronize()
    check(out.float().cpu().numpy(), lse.cpu().numpy(), ref, ref_lse, what="merge")
