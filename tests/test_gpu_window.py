"""GPU parity of the sink + sliding-window verify attention (window > 0 in
sv_verify_params) against the float64 oracle: windows from one position to
ones covering the context, with and without sink positions, forced split
counts (chunks outside the window and sink are skipped by the attention and
the merge), fp16 and FP8 KV, 96 rows per KV head, blocks of a width per
request, and the 512K workload with a 2,048-position window."""
import numpy as np
import pytest
import torch

from helpers import case, check, host, say
from long_context_gqa_amd import binding as B
from long_context_gqa_amd import workloads as W
from oracle import attention as oatt

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run(x, window, sink, splits=0, q_len=None, kv=None, max_kv=None):
    kvl = (kv if kv is not None else x.kv_lens).cuda()
    mk = max_kv if max_kv is not None else int(x.kv_lens.max())
    out, lse, flags = B.verify_attention(x.q, x.k_pages, x.v_pages, x.page_table.cuda(), kvl, q_len or x.wl.q_len, mk,
                                         x.k_scales, x.v_scales, x.sm_scale, splits, window=window, sink=sink)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), int(flags.item())


def oracle_w(x, window, sink, groups=None):
    h = host(x)
    return oatt.verify_attention_window(h["q"], h["k_pages"], h["v_pages"], h["page_table"], h["kv_lens"],
                                        x.wl.q_len, x.sm_scale, window, sink, h["k_scales"], h["v_scales"],
                                        rows=groups)


@pytest.mark.parametrize("kv_dtype", ["fp16", "fp8_e4m3"])
@pytest.mark.parametrize("B_,q,lens,P,Wn,S", [
    (1, 8, [3000], 16, 1, 0),
    (1, 8, [3000], 16, 16, 0),
    (2, 8, [5000, 700], 16, 100, 4),
    (2, 8, [9000, 2100], 64, 2048, 64),
    (3, 5, [40, 1500, 333], 16, 37, 5),
    (1, 16, [4000], 16, 300, 16),      # 96 rows: two row blocks
    (2, 8, [600, 900], 16, 5000, 0),   # covering window: full attention
])
def test_window_parity(B_, q, lens, P, Wn, S, kv_dtype):
    x = case(B_, q, lens, P, "unit", seed=Wn + S + q, kv_dtype=kv_dtype)
    ref, ref_lse = oracle_w(x, Wn, S)
    for splits in (0, 1, 3, 7):
        say(f"B={B_} q={q} lens={lens} P={P} W={Wn} S={S} {kv_dtype} splits={splits}")
        out, lse, flags = run(x, Wn, S, splits)
        assert flags == 0
        check(out, lse, ref, ref_lse, what=f"W={Wn} S={S} splits={splits}")


def test_covering_window_equals_full_attention_bitwise():
    # chunks anchored at absolute positions and masked keys of weight zero:
    # a window that covers every row's context gives the full-attention bits
    x = case(2, 8, [1500, 3100], 16, "unit", seed=4)
    for splits in (0, 5):
        full = run(x, 0, 0, splits)
        win = run(x, 4000, 0, splits)
        assert np.array_equal(full[0], win[0]) and np.array_equal(full[1], win[1])


def test_window_with_widths_per_request():
    widths, prefixes, Wn, S = [3, 8, 1, 6], [900, 4000, 70, 2500], 200, 8
    wl = W.Workload("ragged_window", len(widths), 8, ("fixed", 0), 16, seed=17)
    x = W.make_verify_inputs(wl, "unit", device="cuda", kv_lens=[L + 8 for L in prefixes])
    kv = torch.tensor([L + w for L, w in zip(prefixes, widths)], dtype=torch.int32)
    q = W.pack_rows(x.q, 8, widths)
    qs = W.row_offsets(widths)
    c = B.RaggedVerifyCall(q, qs.cuda(), x.k_pages, x.v_pages, x.page_table.cuda(), kv.cuda(), 8,
                           int(x.kv_lens.max()), sm_scale=x.sm_scale, num_splits=3, window=Wn, sink=S)
    out, lse = c.run()
    torch.cuda.synchronize()
    h = host(x)
    for b, wdt in enumerate(widths):
        r0, r1 = int(qs[b]), int(qs[b + 1])
        ro, rl = oatt.verify_attention_window(q[r0:r1].cpu(), h["k_pages"], h["v_pages"], h["page_table"][b:b + 1],
                                              kv[b:b + 1], wdt, x.sm_scale, Wn, S)
        check(out[r0:r1].float().cpu().numpy(), lse[r0:r1].cpu().numpy(), ro, rl, what=f"request {b}")


def test_512k_window_2048_sink_4_sampled():
    wl = W.WORKLOADS[3]
    x = W.make_verify_inputs(wl, "unit", device="cuda")
    out, lse, flags = run(x, 2048, 4)
    assert flags == 0
    groups = [(0, 0), (0, 3)]
    ref, ref_lse = oracle_w(x, 2048, 4, groups)
    from helpers import rows_of
    check(out, lse, ref, ref_lse, mask=rows_of(x, groups), what="512K W=2048 S=4")
