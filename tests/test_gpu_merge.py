"""GPU sv_verify_merge against the oracle's merge on arbitrary partials:
many splits, empty splits (lse = -inf), fully empty rows, head_dim values
that are not 256, and both kernels (a workgroup per (row, head) item for
few items, a wave per item from 4,096 items)."""
import numpy as np
import pytest
import torch

from helpers import say
from long_context_gqa_amd import binding as B
from oracle import attention as oatt

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("S,R,H,D", [(1, 3, 2, 256), (5, 4, 3, 100), (130, 2, 24, 256), (17, 3, 2, 1024),
                                     (300, 1, 1, 4), (300, 2, 1, 4),
                                     # up to 64 splits of 256 channels: every load in one round trip
                                     (64, 8, 24, 256), (63, 2, 3, 256), (33, 8, 24, 256), (2, 5, 24, 256),
                                     (65, 2, 3, 256),
                                     # 4,096 and more (row, head) items: one wave per item
                                     (7, 200, 24, 256), (20, 171, 24, 256), (3, 4096, 1, 100), (1, 512, 24, 256)])
def test_merge_matches_oracle(S, R, H, D):
    # order-one partials (each split's normalised output, N(0,1)); the merged
    # row is a convex combination of them, so it is of order one as well
    g = torch.Generator().manual_seed(S * 7 + D)
    po = torch.randn((S, R, H, D), generator=g)
    pl = torch.randn((S, R, H), generator=g) * 3
    drop = torch.rand((S, R, H), generator=g) < 0.3
    pl[drop] = -float("inf")
    po[drop] = 0.0
    pl[:, 0, 0] = -float("inf")  # one row with every split empty
    po[:, 0, 0] = 0.0
    ref, ref_lse = oatt.merge_partials(po.numpy(), pl.numpy())
    out = torch.empty((R, H, D), dtype=torch.float16, device="cuda")
    lse = torch.empty((R, H), dtype=torch.float32, device="cuda")
    B.sv_verify_merge(po.cuda(), pl.cuda(), out, lse)
    torch.cuda.synchronize()
    o, l = out.float().cpu().numpy(), lse.cpu().numpy()
    err = np.abs(o - ref).max()
    # the merge's own error: the fp16 rounding of the result (half an ulp of
    # the reference's fp16 value) plus fp32 rounding in the weights and sums
    ulp = np.spacing(np.abs(ref.astype(np.float16))).astype(np.float64)
    past = (np.abs(o - ref) - 0.5 * ulp - 1e-5 * np.abs(po.numpy()).max()).max()
    say(f"S={S} R={R} H={H} D={D}: max|err| {err:.2e}  max|ref| {np.abs(ref).max():.2f}  "
        f"beyond half an ulp + fp32 bound {past:.2e}")
    assert err <= 2e-3
    assert past <= 0
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(l))
    if fin.any():
        assert np.abs(l[fin] - ref_lse[fin]).max() <= 1e-4
    assert (o[0, 0] == 0).all()
