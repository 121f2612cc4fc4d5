"""GPU parity of extend chunks (q_len above the verify block sizes: new
tokens processed on top of a cached prefix, causally, in one call) against
the float64 oracle: 17 to 512 rows per request, up to 8192 rows on one KV
head (the workgroups of one key chunk then split the rows into many tiles
of up to 48), fp16 and FP8 KV, forced and automatic splits, a pure prefill
with no prefix, extend chunks mixed with verify blocks in one ragged batch,
and an extend chunk under a sliding window."""
import numpy as np
import pytest
import torch

from helpers import case, check, host, run_gpu, say
from long_context_gqa_amd import binding as B
from long_context_gqa_amd import workloads as W
from oracle import attention as oatt

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("q,lens,P,kv_dtype,splits,Hq,Hkv", [
    (17, [300, 1000], 16, "fp16", 0, 24, 4),       # 102 rows per KV head: 3 tiles
    (32, [2000], 64, "fp8_e4m3", 3, 24, 4),
    (64, [5000, 70], 16, "fp16", 0, 24, 4),        # second request: 6 prefix positions
    (100, [3000], 48, "fp8_e4m3", 5, 24, 4),
    (256, [4096], 16, "fp16", 0, 24, 4),
    (512, [1500], 32, "fp16", 2, 24, 4),
    (512, [600], 16, "fp8_e4m3", 0, 16, 1),        # 8192 rows on one KV head
    (40, [40, 41], 16, "fp16", 0, 24, 4),          # a prefill with no prefix (and one of one position)
])
def test_extend_matches_oracle(q, lens, P, kv_dtype, splits, Hq, Hkv):
    say(f"q={q} lens={lens} P={P} {kv_dtype} splits={splits} Hq={Hq} Hkv={Hkv}")
    x = case(len(lens), q, lens, P, kv_dtype=kv_dtype, Hq=Hq, Hkv=Hkv, seed=q + len(lens))
    out, lse, flags = run_gpu(x, num_splits=splits)
    assert flags == 0
    h = host(x)
    ref, ref_lse = oatt.verify_attention(h["q"], h["k_pages"], h["v_pages"], h["page_table"], h["kv_lens"], q,
                                         x.sm_scale, h["k_scales"], h["v_scales"])
    check(out, lse, ref, ref_lse, what=f"q={q}")


def test_extend_chunks_and_verify_blocks_in_one_batch():
    widths, prefixes = [3, 120, 16, 0, 64], [900, 2500, 4000, 100, 0]
    qmax = max(widths)
    wl = W.Workload("mixed", len(widths), qmax, ("fixed", 0), 16, seed=31)
    x = W.make_verify_inputs(wl, "unit", device="cuda", kv_lens=[L + qmax for L in prefixes])
    kv = torch.tensor([L + w for L, w in zip(prefixes, widths)], dtype=torch.int32)
    q = W.pack_rows(x.q, qmax, widths)
    qs = W.row_offsets(widths)
    c = B.RaggedVerifyCall(q, qs.cuda(), x.k_pages, x.v_pages, x.page_table.cuda(), kv.cuda(), qmax,
                           int(x.kv_lens.max()), sm_scale=x.sm_scale)
    out, lse = c.run()
    torch.cuda.synchronize()
    assert int(c.flags.item()) == 0
    h = host(x)
    for b, wdt in enumerate(widths):
        if wdt == 0:
            continue
        r0, r1 = int(qs[b]), int(qs[b + 1])
        ro, rl = oatt.verify_attention(q[r0:r1].cpu(), h["k_pages"], h["v_pages"], h["page_table"][b:b + 1],
                                       kv[b:b + 1], wdt, x.sm_scale)
        check(out[r0:r1].float().cpu().numpy(), lse[r0:r1].cpu().numpy(), ro, rl, what=f"request {b} width {wdt}")


@pytest.mark.parametrize("kv_dtype", ["fp16", "fp8_e4m3"])
def test_extend_under_a_sliding_window(kv_dtype):
    q, lens, Wn, S = 128, [3000, 200], 256, 4
    x = case(len(lens), q, lens, 16, kv_dtype=kv_dtype, seed=5)
    out, lse, flags = B.verify_attention(x.q, x.k_pages, x.v_pages, x.page_table.cuda(), x.kv_lens.cuda(), q,
                                         int(x.kv_lens.max()), x.k_scales, x.v_scales, x.sm_scale, 0,
                                         window=Wn, sink=S)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    h = host(x)
    ref, ref_lse = oatt.verify_attention_window(h["q"], h["k_pages"], h["v_pages"], h["page_table"], h["kv_lens"], q,
                                                x.sm_scale, Wn, S, h["k_scales"], h["v_scales"])
    check(out.float().cpu().numpy(), lse.cpu().numpy(), ref, ref_lse, what=f"window {Wn} sink {S}")
