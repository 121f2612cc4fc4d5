"""A whole verify step (attention, merge, greedy accept) captured once in a HIP
graph and replayed with new device-resident inputs: the cache lengths, the
queries, the logits and the drafts change in place between replays (the host
only ever passes its fixed bound max_kv_len, as a serving loop that captures
verify with max-context metadata does). Every replay must equal an eager call
on the same inputs bit for bit, and one replay is also checked against the
float64 oracle. The graph's own flag reset is a fill kernel (no memset node)."""
import numpy as np
import pytest
import torch

from helpers import case, check, host, say
from long_context_gqa_amd import binding as B
from long_context_gqa_amd import workloads as W
from oracle import accept as oacc
from oracle import attention as oatt

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("kv_dtype", ["fp16", "fp8_e4m3"])
def test_verify_step_replays_with_new_lengths_and_inputs(kv_dtype):
    lens0 = [20000, 9000, 24000, 513]
    q_len, Bn = 8, len(lens0)
    x = case(Bn, q_len, lens0, 16, kv_dtype=kv_dtype, seed=61)
    max_kv = max(lens0)
    wl = W.Workload("graph", Bn, q_len, ("fixed", 0), 16, kv_dtype=kv_dtype, seed=62, vocab=50_000)
    acc_in = W.make_accept_inputs(wl, device="cuda")
    dev = torch.device("cuda")
    q = x.q.clone()
    kv = torch.tensor(lens0, dtype=torch.int32, device=dev)
    table = x.page_table.to(dev).contiguous()
    logits, drafts = acc_in.logits.clone(), acc_in.draft_ids.clone()

    call = B.VerifyCall(q, x.k_pages, x.v_pages, table, kv, q_len, max_kv, x.k_scales, x.v_scales, x.sm_scale)
    acall = B.AcceptCall(logits, drafts, q_len, kv)
    say(f"{kv_dtype}: {call.splits} splits x {call.chunk} tokens")

    def step():
        call.flags.zero_()
        call.run()
        acall.run()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    rng = np.random.default_rng(63)
    # each request's pages hold at most its first length; every length >= q_len
    for r, lens in enumerate([lens0, [19000, 8, 23999, 100], [513, 9000, 16, 500], [20000, 8999, 24000, 8]]):
        kv.copy_(torch.tensor(lens, dtype=torch.int32))
        q.copy_((torch.randn(q.shape, generator=torch.Generator().manual_seed(100 + r)) / 16).to(torch.float16))
        planted = [int(v) for v in rng.integers(0, q_len, Bn)]
        acc_r = W.make_accept_inputs(wl, device="cuda", planted=planted)
        logits.copy_(acc_r.logits)
        drafts.copy_(acc_r.draft_ids)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [call.out.clone(), call.out_lse.clone(), acall.accept_len.clone(), acall.bonus.clone(),
               acall.kv_out.clone(), int(call.flags.item())]
        # the same inputs through eager calls with their own buffers
        ec = B.VerifyCall(q, x.k_pages, x.v_pages, table, kv, q_len, max_kv, x.k_scales, x.v_scales, x.sm_scale)
        ea = B.AcceptCall(logits, drafts, q_len, kv)
        ec.run()
        ea.run()
        torch.cuda.synchronize()
        say(f"  replay {r}: lengths {lens}, planted {planted}, accepted {got[2].tolist()}")
        assert got[5] == 0
        assert torch.equal(got[0], ec.out) and torch.equal(got[1], ec.out_lse)
        assert torch.equal(got[2], ea.accept_len) and torch.equal(got[3], ea.bonus) and torch.equal(got[4], ea.kv_out)
        assert got[2].cpu().tolist() == planted
        assert got[4].cpu().tolist() == [n - q_len + 1 + a for n, a in zip(lens, planted)]
        if r == 1:
            h = host(x)
            h["q"] = q.cpu()
            ref, ref_lse = oatt.verify_attention(h["q"], h["k_pages"], h["v_pages"], h["page_table"],
                                                 torch.tensor(lens, dtype=torch.int32), q_len, x.sm_scale,
                                                 h["k_scales"], h["v_scales"])
            check(got[0].float().cpu().numpy(), got[1].cpu().numpy(), ref, ref_lse, what=f"replay {r}")
            a_ref, b_ref, _, _ = oacc.greedy_accept(logits.cpu().numpy(), drafts.cpu().numpy(), q_len)
            assert got[2].cpu().tolist() == list(a_ref) and got[3].cpu().tolist() == list(b_ref)
