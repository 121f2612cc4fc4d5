"""GPU parity of sv_verify_attention (through the C ABI) against the float64
oracle, and the invariants the verify step must satisfy: q = 1 equals decode,
row i equals decode over the prefix plus drafts[:i], split-count and
page-permutation invariance, one-hot position probes, poisoned slots."""
import numpy as np
import pytest
import torch

from helpers import case, check, host, oracle, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("variant", ["unit", "literal"])
@pytest.mark.parametrize("B,q_len,lens,P", [
    (1, 1, [1], 16),
    (1, 1, [77], 16),
    (1, 2, [2], 16),
    (1, 3, [200], 16),
    (1, 8, [8], 16),
    (1, 8, [4104], 16),
    (2, 8, [333, 1290], 64),
    (3, 5, [17, 160, 1025], 16),
    (1, 16, [321], 16),            # q-group 16 at KV length 321
    (2, 16, [16, 2500], 64),
    (3, 11, [64, 65, 900], 32),
])
def test_small_parity(B, q_len, lens, P, variant):
    x = case(B, q_len, lens, P, variant, seed=B * 100 + q_len)
    ref, ref_lse = oracle(x)
    for splits in (0, 1, 2, 3, 7):
        say(f"B={B} q={q_len} lens={lens} P={P} {variant} splits={splits}")
        out, lse, flags = run_gpu(x, num_splits=splits)
        assert flags == 0
        check(out, lse, ref, ref_lse, what=f"splits={splits}")


def test_causal_offsets_sweep():
    # every prefix length 0..333 behind a block of 4 (kv_len - q = offset)
    for L in list(range(0, 40)) + [63, 64, 65, 127, 128, 129, 200, 255, 256, 257, 300, 333]:
        x = case(1, 4, [L + 4], 16, "unit", seed=L)
        ref, ref_lse = oracle(x)
        out, lse, _ = run_gpu(x, num_splits=0 if L % 2 else 3)
        check(out, lse, ref, ref_lse, what=f"L={L}")


def test_split_count_invariance():
    x = case(2, 8, [3000, 5000], 16, "unit", seed=5)
    ref, ref_lse = oracle(x)
    outs = []
    for splits in (1, 2, 3, 7, 64, 0):
        out, lse, _ = run_gpu(x, num_splits=splits)
        check(out, lse, ref, ref_lse, what=f"splits={splits}")
        outs.append(out)
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2e-3


def test_q1_equals_decode_and_rows_equal_decode_over_prefix():
    L, q_len = 2000, 8
    x = case(1, q_len, [L + q_len], 16, "unit", seed=11)
    out, lse, _ = run_gpu(x)
    ref, ref_lse = oracle(x)
    check(out, lse, ref, ref_lse, what="verify block")
    for i in range(q_len):
        # the same cache and page table, a one-row block ending at position L+i
        xi = case(1, 1, [L + i + 1], 16, "unit", seed=11)
        xi.k_pages, xi.v_pages, xi.page_table = x.k_pages, x.v_pages, x.page_table
        xi.q = x.q[i:i + 1].contiguous()
        oi, li, _ = run_gpu(xi, max_kv_len=L + q_len)
        # GPU decode vs the oracle's row i of the verify block
        check(oi, li, ref[i:i + 1], ref_lse[i:i + 1], what=f"decode row {i}")
        # and verify row i vs GPU decode: bitwise (chunks are anchored at
        # absolute positions and masked keys weigh exactly zero)
        same = np.array_equal(oi[0], out[i])
        say(f"  row {i} bitwise equal to decode: {same}")
        assert np.abs(oi[0] - out[i]).max() <= 2e-3


def test_page_permutation_invariance_bitwise():
    x = case(2, 8, [700, 1500], 16, "unit", seed=3)
    out, lse, _ = run_gpu(x)
    # move every physical page to a new slot and rewrite the table
    n = x.k_pages.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(1))
    inv = torch.argsort(perm)
    x2 = case(2, 8, [700, 1500], 16, "unit", seed=3)
    x2.k_pages = x.k_pages[perm.cuda()].contiguous()
    x2.v_pages = x.v_pages[perm.cuda()].contiguous()
    t = x.page_table.clone()
    t[t >= 0] = inv[t[t >= 0].long()].to(torch.int32)
    x2.page_table = t
    out2, lse2, _ = run_gpu(x2)
    assert np.array_equal(out, out2)
    assert np.array_equal(lse, lse2)


def test_one_hot_position_probe_is_exact():
    # Q = 8u, the planted key = 8u, all other keys 0: the planted logit is
    # 1024 above the rest, so the output row is exactly that key's V row.
    L, q_len, P = 300, 8, 16
    x = case(1, q_len, [L + q_len], P, "unit", seed=2)
    g = torch.Generator().manual_seed(4)
    u = (torch.randint(0, 2, (4, 256), generator=g) * 2 - 1).to(torch.float16)
    x.q.copy_((8 * u).repeat_interleave(6, 0).unsqueeze(0).expand(q_len, 24, 256).cuda())
    kp = x.k_pages
    pt = x.page_table[0]
    valid = kp.clone()
    valid.zero_()
    for t_star in (0, 15, 16, 299, 300, 301, 303, 307):
        kp = valid.clone()
        for gq in range(4):
            t = (t_star + 37 * gq) % (L + q_len)
            kp[int(pt[t // P]), gq, t % P] = (8 * u[gq]).cuda()
        x.k_pages = kp
        out, lse, _ = run_gpu(x)
        h = host(x)
        ref, ref_lse = oracle(x, h=h)
        check(out, lse, ref, ref_lse, what=f"probe t*={t_star}")
        for i in range(q_len):
            for gq in range(4):
                t = (t_star + 37 * gq) % (L + q_len)
                if t <= L + i:
                    vrow = x.v_pages[int(pt[t // P]), gq, t % P].float().cpu().numpy()
                    assert np.array_equal(out[i, 6 * gq], vrow)


def test_bad_page_ids_and_lengths_are_flagged_and_clamped():
    x = case(2, 8, [200, 300], 16, "unit", seed=9)
    t = x.page_table.clone()
    t[1, 3] = 10 ** 6  # outside the pool: page 0 is read instead, the flag is set
    out, lse, flags = run_gpu(x, page_table=t)
    assert flags & 4
    assert np.isfinite(out[:8]).all()
    kv = x.kv_lens.clone()
    kv[0] = 5  # shorter than the block
    out, lse, flags = run_gpu(x, kv_lens=kv, max_kv_len=300)
    assert flags & 2
    kv = x.kv_lens.clone()
    kv[1] = 400  # above the host bound max_kv_len
    out, lse, flags = run_gpu(x, kv_lens=kv, max_kv_len=300)
    assert flags & 1


# ---------------------------------------------------------------------------
# FP8 E4M3 KV with per-token, per-KV-head fp16 scales over 64-channel blocks

@pytest.mark.parametrize("variant", ["unit", "literal"])
@pytest.mark.parametrize("B,q_len,lens,P", [
    (1, 1, [77], 16),
    (1, 8, [8], 16),
    (2, 8, [333, 1290], 16),
    (3, 5, [17, 160, 1025], 64),
    (1, 8, [5000], 32),
])
def test_fp8_small_parity(B, q_len, lens, P, variant):
    x = case(B, q_len, lens, P, variant, seed=B * 31 + q_len, kv_dtype="fp8_e4m3")
    ref, ref_lse = oracle(x)
    for splits in (0, 1, 3):
        say(f"fp8 B={B} q={q_len} lens={lens} P={P} {variant} splits={splits}")
        out, lse, flags = run_gpu(x, num_splits=splits)
        assert flags == 0
        check(out, lse, ref, ref_lse, what=f"fp8 splits={splits}")


def test_fp8_every_code_is_decoded_exactly():
    # K and V cycle through every finite E4M3 code (subnormals included) with
    # random scales; the oracle decodes from the format definition
    x = case(1, 8, [1200], 16, "unit", seed=77, kv_dtype="fp8_e4m3")
    g = torch.Generator().manual_seed(5)
    codes = torch.tensor([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=torch.uint8)
    n = x.k_pages.numel()
    kc = codes[torch.randint(0, len(codes), (n,), generator=g)].view(x.k_pages.shape)
    vc = codes[torch.arange(n) % len(codes)].view(x.v_pages.shape)
    x.k_pages = kc.cuda()
    x.v_pages = vc.cuda()
    ks = (torch.rand(x.k_scales.shape, generator=g) * 0.004 + 1e-4).to(torch.float16)
    vs = (torch.rand(x.v_scales.shape, generator=g) * 0.004 + 1e-4).to(torch.float16)
    x.k_scales, x.v_scales = ks.cuda(), vs.cuda()
    ref, ref_lse = oracle(x)
    out, lse, _ = run_gpu(x, num_splits=2)
    check(out, lse, ref, ref_lse, what="fp8 every code")


def test_fp8_one_hot_probe_is_exact():
    # one key per KV head equal to the query direction; the output row must be
    # the dequantised V row of that key exactly (its fp16 rounding)
    L, q_len, P = 200, 8, 16
    x = case(1, q_len, [L + q_len], P, "unit", seed=3, kv_dtype="fp8_e4m3")
    g = torch.Generator().manual_seed(6)
    u = (torch.randint(0, 2, (4, 256), generator=g) * 2 - 1).to(torch.float16)
    x.q.copy_((8 * u).repeat_interleave(6, 0).unsqueeze(0).expand(q_len, 24, 256).cuda())
    kp = torch.zeros_like(x.k_pages)
    ks = torch.ones_like(x.k_scales)
    pt = x.page_table[0]
    t_star = 123
    code8 = torch.where(u > 0, torch.tensor(0x48, dtype=torch.uint8), torch.tensor(0xC8, dtype=torch.uint8))  # +-4
    for gq in range(4):
        kp[int(pt[t_star // P]), gq, t_star % P] = code8[gq].cuda()
    x.k_pages, x.k_scales = kp, ks
    out, lse, _ = run_gpu(x)
    ref, ref_lse = oracle(x)
    check(out, lse, ref, ref_lse, what="fp8 probe")
    for i in range(q_len):
        for gq in range(4):
            want = ref[i, 6 * gq].astype(np.float16).astype(np.float32)
            assert np.array_equal(out[i, 6 * gq], want)


@pytest.mark.parametrize("kv_dtype", ["fp16", "fp8_e4m3"])
@pytest.mark.parametrize("Hq,q_len", [(16, 16), (20, 16), (24, 16), (24, 12)])
def test_more_than_48_rows_two_row_blocks(kv_dtype, Hq, q_len):
    # 64, 80, 96 and 72 rows per KV head: two workgroups of up to 48 rows
    # read the same keys; ragged lengths, split and unsplit
    x = case(3, q_len, [q_len + 5, 1000, 2333], 16, "unit", seed=Hq + q_len, kv_dtype=kv_dtype, Hq=Hq, Hkv=4)
    ref, ref_lse = oracle(x)
    for splits in (1, 0, 5):
        say(f"{kv_dtype} Hq={Hq} q={q_len} rows={q_len * Hq // 4} splits={splits}")
        out, lse, flags = run_gpu(x, num_splits=splits)
        assert flags == 0
        check(out, lse, ref, ref_lse, what=f"{q_len * Hq // 4} rows splits={splits}")
