"""A seeded sweep of shapes against the float64 oracle, over the envelope
the ABI accepts: query groups of 1..12 heads per KV head with up to 8 KV
heads (rows per KV head up to 96), page sizes that are and are not powers of
two (16..4096), fp16 and FP8 KV, forced and automatic split counts, sliding
windows with sinks, and blocks of a width per request; and shapes that the
planner gives the two-half kernel (49 to 96 rows per KV head with fp16 keys
over a pass of 32 MB or more, forced split counts), each asserted through
sv_verify_plan_kernel before the call."""
import numpy as np
import pytest
import torch

from helpers import check, host, say
from long_context_gqa_amd import binding as B
from long_context_gqa_amd import workloads as W
from oracle import attention as oatt

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def draw_shape(rng):
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 12]))
    q = int(rng.integers(1, min(16, 96 // G) + 1))
    Bn = int(rng.integers(1, 4))
    P = int(rng.choice([16, 32, 48, 64, 80, 128, 256, 4096]))
    lens = [int(rng.integers(q, 5000)) for _ in range(Bn)]
    kv_dtype = str(rng.choice(["fp16", "fp8_e4m3"]))
    splits = int(rng.choice([0, 0, 1, 2, 5, 9]))
    window = int(rng.choice([0, 0, 0, 1, 33, 700]))
    sink = int(rng.choice([0, 4, 100])) if window else 0
    return Hkv, G, q, Bn, P, lens, kv_dtype, splits, window, sink


@pytest.mark.parametrize("seed", range(24))
def test_random_shape(seed):
    rng = np.random.default_rng(4242 + seed)
    Hkv, G, q, Bn, P, lens, kv_dtype, splits, window, sink = draw_shape(rng)
    say(f"seed {seed}: Hkv={Hkv} G={G} q={q} B={Bn} P={P} lens={lens} {kv_dtype} splits={splits} "
        f"window={window} sink={sink}")
    wl = W.Workload("sweep", Bn, q, ("fixed", 0), P, kv_dtype=kv_dtype, seed=seed + 77, num_q_heads=Hkv * G,
                    num_kv_heads=Hkv)
    x = W.make_verify_inputs(wl, "unit", device="cuda", kv_lens=lens)
    out, lse, flags = B.verify_attention(x.q, x.k_pages, x.v_pages, x.page_table.cuda(), x.kv_lens.cuda(), q,
                                         int(x.kv_lens.max()), x.k_scales, x.v_scales, x.sm_scale, splits,
                                         window=window, sink=sink)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    h = host(x)
    ref, ref_lse = oatt.verify_attention_window(h["q"], h["k_pages"], h["v_pages"], h["page_table"], h["kv_lens"], q,
                                                x.sm_scale, window, sink, h["k_scales"], h["v_scales"])
    check(out.float().cpu().numpy(), lse.cpu().numpy(), ref, ref_lse, what=f"seed {seed}")


@pytest.mark.parametrize("seed", range(8))
def test_random_widths_per_request(seed):
    rng = np.random.default_rng(9000 + seed)
    Hkv, G, qmax, Bn, P, lens, kv_dtype, splits, window, sink = draw_shape(rng)
    Bn = int(rng.integers(2, 6))
    widths = [int(rng.integers(0, qmax + 1)) for _ in range(Bn)]
    if sum(widths) == 0:
        widths[0] = qmax
    prefixes = [int(rng.integers(0, 4000)) for _ in range(Bn)]
    say(f"seed {seed}: Hkv={Hkv} G={G} widths={widths} P={P} {kv_dtype} splits={splits} window={window} "
        f"sink={sink}")
    wl = W.Workload("sweep_ragged", Bn, qmax, ("fixed", 0), P, kv_dtype=kv_dtype, seed=seed + 99,
                    num_q_heads=Hkv * G, num_kv_heads=Hkv)
    x = W.make_verify_inputs(wl, "unit", device="cuda", kv_lens=[L + qmax for L in prefixes])
    kv = torch.tensor([L + w for L, w in zip(prefixes, widths)], dtype=torch.int32)
    q = W.pack_rows(x.q, qmax, widths)
    qs = W.row_offsets(widths)
    c = B.RaggedVerifyCall(q, qs.cuda(), x.k_pages, x.v_pages, x.page_table.cuda(), kv.cuda(), qmax,
                           int(x.kv_lens.max()), x.k_scales, x.v_scales, x.sm_scale, splits, window=window, sink=sink)
    out, lse = c.run()
    torch.cuda.synchronize()
    assert int(c.flags.item()) == 0
    h = host(x)
    for b, wdt in enumerate(widths):
        if wdt == 0:
            continue
        r0, r1 = int(qs[b]), int(qs[b + 1])
        ro, rl = oatt.verify_attention_window(q[r0:r1].cpu(), h["k_pages"], h["v_pages"], h["page_table"][b:b + 1],
                                              kv[b:b + 1], wdt, x.sm_scale, window, sink,
                                              h["k_scales"], h["v_scales"])
        check(out[r0:r1].float().cpu().numpy(), lse[r0:r1].cpu().numpy(), ro, rl, what=f"request {b}")


def draw_two_half_shape(rng):
    """A shape the planner gives the two-half kernel under a forced split
    count: 49 to 96 rows per KV head, fp16 keys, a pass of 32 MB or more."""
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([4, 6, 8, 12]))
    q = int(rng.integers(48 // G + 1, 96 // G + 1))
    Bn = int(rng.integers(1, 4))
    P = int(rng.choice([16, 32, 48, 64, 80, 256, 4096]))
    need = -(-32768 // (Bn * Hkv))  # positions per request for 32 MB (1 KB of K and V per position and KV head)
    lens = [int(rng.integers(q, need + 6000)) for _ in range(Bn)]
    lens[int(rng.integers(0, Bn))] = int(rng.integers(need, need + 6000))
    window = int(rng.choice([0, 0, 0, need + 300]))
    sink = int(rng.choice([0, 16, 64])) if window else 0
    live = min(max(lens), sink + window + q + 48) if window else max(lens)
    splits = int(rng.choice([s for s in (1, 2, 3, 5, 9, 17) if -(-live // s) <= 32768]))
    return Hkv, G, q, Bn, P, lens, splits, window, sink


@pytest.mark.parametrize("seed", range(12))
def test_random_two_half_shape(seed):
    rng = np.random.default_rng(6100 + seed)
    Hkv, G, q, Bn, P, lens, splits, window, sink = draw_two_half_shape(rng)
    ragged = seed % 3 == 2
    say(f"seed {seed}: Hkv={Hkv} G={G} q={q} B={Bn} P={P} lens={lens} splits={splits} window={window} "
        f"sink={sink} ragged={ragged}")
    wl = W.Workload("sweep_halves", Bn, q, ("fixed", 0), P, seed=seed + 55, num_q_heads=Hkv * G, num_kv_heads=Hkv)
    x = W.make_verify_inputs(wl, "unit", device="cuda", kv_lens=lens)
    h = host(x)
    if ragged:
        widths = [int(rng.integers(0, q + 1)) for _ in range(Bn)]
        widths[0] = q
        kv = torch.tensor([L - q + w for L, w in zip(lens, widths)], dtype=torch.int32)
        qp = W.pack_rows(x.q, q, widths)
        qs = W.row_offsets(widths)
        c = B.RaggedVerifyCall(qp, qs.cuda(), x.k_pages, x.v_pages, x.page_table.cuda(), kv.cuda(), q,
                               int(x.kv_lens.max()), None, None, x.sm_scale, splits, window=window, sink=sink)
        assert c.kernel == B.SV_KERNEL_TWO_HALVES
        out, lse = c.run()
        torch.cuda.synchronize()
        assert int(c.flags.item()) == 0
        for b, wdt in enumerate(widths):
            if wdt == 0:
                continue
            r0, r1 = int(qs[b]), int(qs[b + 1])
            ro, rl = oatt.verify_attention_window(qp[r0:r1].cpu(), h["k_pages"], h["v_pages"],
                                                  h["page_table"][b:b + 1], kv[b:b + 1], wdt, x.sm_scale, window,
                                                  sink, None, None)
            check(out[r0:r1].float().cpu().numpy(), lse[r0:r1].cpu().numpy(), ro, rl,
                  what=f"seed {seed} request {b}")
        return
    else:
        c = B.VerifyCall(x.q, x.k_pages, x.v_pages, x.page_table.cuda(), x.kv_lens.cuda(), q, int(x.kv_lens.max()),
                         None, None, x.sm_scale, splits, window=window, sink=sink)
        assert c.kernel == B.SV_KERNEL_TWO_HALVES
        out, lse = c.run()
        torch.cuda.synchronize()
        assert int(c.flags.item()) == 0
        ref, ref_lse = oatt.verify_attention_window(h["q"], h["k_pages"], h["v_pages"], h["page_table"],
                                                    h["kv_lens"], q, x.sm_scale, window, sink, None, None)
    check(out.float().cpu().numpy(), lse.cpu().numpy(), ref, ref_lse, what=f"seed {seed}")
