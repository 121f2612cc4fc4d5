"""The full-size workloads (4K, 8 x 32K, 512K with biased keys, ragged
8K-131K DFlash blocks of 16) through the launch configuration the benchmark
times, checked against the oracle on sampled (request, KV head) groups, in
both value variants; plus the GPU merge fed oracle partials."""
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


def sample_groups(wl, kv_lens):
    B_ = wl.batch
    if B_ == 1:
        return [(0, 0), (0, wl.num_kv_heads - 1)]
    lens = list(kv_lens)
    picks = {int(np.argmin(lens)), int(np.argmax(lens)), B_ // 2}
    return [(b, (b * 3) % wl.num_kv_heads) for b in sorted(picks)]


@pytest.mark.parametrize("variant", ["literal", "unit"])
@pytest.mark.parametrize("wl_id", [1, 2, 3, 4, 5])
def test_full_size_config(wl_id, variant):
    wl = W.WORKLOADS[wl_id]
    say(f"config {wl_id} {wl.name} {variant}: generating")
    x = W.make_verify_inputs(wl, variant, device="cuda")
    say(f"  pool {tuple(x.k_pages.shape)}, max kv {x.max_kv_len}")
    out, lse, flags = run_gpu(x)
    assert flags == 0
    assert np.isfinite(out).all()
    groups = sample_groups(wl, x.kv_lens.tolist())
    say(f"  oracle on groups {groups}")
    ref, ref_lse = oracle(x, groups=groups)
    check(out, lse, ref, ref_lse, mask=rows_of(x, groups), what=f"config {wl_id} {variant}")
    del x
    torch.cuda.empty_cache()


def test_512k_split_count_invariance_sampled():
    wl = W.WORKLOADS[3]
    x = W.make_verify_inputs(wl, "unit", device="cuda")
    groups = [(0, 1)]
    ref, ref_lse = oracle(x, groups=groups)
    mask = rows_of(x, groups)
    outs = []
    for splits in (0, 16, 97, 300):
        out, lse, _ = run_gpu(x, num_splits=splits)
        check(out, lse, ref, ref_lse, mask=mask, what=f"512K splits={splits}")
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
