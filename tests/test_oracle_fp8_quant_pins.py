"""Pins of the FP8 quantiser oracle (appending rows to an E4M3 cache) against
facts outside it: every finite code encodes back to itself, the nearest value
by brute force with ties to the even code, torch's float8_e4m3fn cast on
random values, the closed form that each block's largest |x| lands on 448,
the rounding bound, and the zero-block and sign rules. Planted mistakes (ties
away from zero, a scale from amax / 240) fail them."""
import numpy as np
import pytest
import torch

from oracle import block as oblk
from oracle import fp8

FIN = np.array([c for c in range(256) if np.isfinite(fp8.e4m3_value(c))], dtype=np.uint8)


def test_every_finite_code_encodes_back_to_itself():
    v = fp8.e4m3_decode(FIN)
    assert (fp8.e4m3_encode(v) == FIN).all()  # -0.0 is 0x80, +0.0 is 0x00


def test_nearest_value_by_brute_force_and_ties_to_even():
    rng = np.random.default_rng(0)
    y = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-0.02, 0.02, 5000)])
    vals = fp8.e4m3_decode(FIN)
    got = fp8.e4m3_decode(fp8.e4m3_encode(y))
    best = np.abs(y[:, None] - vals[None, :]).min(axis=1)
    assert np.array_equal(np.abs(y - got), best)
    # exact midpoints between neighbouring positive values go to the even code
    pos = np.sort(np.unique(vals[vals > 0]))
    mid = (pos[:-1] + pos[1:]) / 2
    codes = fp8.e4m3_encode(mid)
    assert (codes % 2 == 0).all()
    assert (fp8.e4m3_encode(-mid) == (codes | 0x80)).all()


def test_agrees_with_the_library_cast():
    g = torch.Generator().manual_seed(1)
    y = (torch.rand(100000, generator=g) * 2 - 1) * 448
    y = torch.cat([y, torch.randn(20000, generator=g) * 1e-3])
    lib = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.e4m3_encode(y.double().numpy()), lib)


def test_quantised_blocks_closed_forms_and_bound():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((50, 4, 256)) * rng.choice([1e-3, 1.0, 300.0], (50, 4, 1))).astype(np.float16)
    x[0, 0, :64] = 0.0                   # an all-zero block: scale 1, codes 0
    x[1, 0, 64:128] = -0.0               # negative zeros: code 0x80
    codes, sc = fp8.quantize_rows(x)
    assert sc[0, 0, 0] == 1.0 and (codes[0, 0, :64] == 0).all()
    assert sc[1, 0, 1] == 1.0 and (codes[1, 0, 64:128] == 0x80).all()
    blocks = np.abs(x.astype(np.float64)).reshape(50, 4, 4, 64).max(-1)
    nz = blocks > 0
    # the largest |x| of a block lands on 448 (code 0x7E up to sign)
    cmax = (codes.reshape(50, 4, 4, 64) & 0x7F).max(-1)
    assert (cmax[nz] == 0x7E).all()
    # dequantised within half a unit in the last place (E4M3 step 2^-3 relative, 2^-9 subnormal)
    deq = fp8.dequantize(codes, sc)
    y = np.abs(x.astype(np.float64)) / np.repeat(sc.astype(np.float64), 64, -1)
    step = np.where(y >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(y, 1e-30))) - 3), 2.0 ** -9)
    bound = (step / 2) * (1 + 1e-6) * np.repeat(sc.astype(np.float64), 64, -1) + 1e-12
    assert (np.abs(deq - x.astype(np.float64)) <= bound).all()


def test_append_fp8_writes_quantised_rows_into_their_slots():
    rng = np.random.default_rng(3)
    pages = rng.integers(0, 256, (6, 2, 4, 128)).astype(np.uint8)
    scales = rng.random((6, 2, 4, 2)).astype(np.float16)
    new = rng.standard_normal((3, 2, 128)).astype(np.float16)
    slots = np.array([5, 17, 8])
    out, osc = oblk.append_kv_fp8(pages, scales, slots, new)
    codes, sc = fp8.quantize_rows(new)
    for r, s in enumerate(slots):
        assert (out[s // 4, :, s % 4] == codes[r]).all() and (osc[s // 4, :, s % 4] == sc[r]).all()
    touched = {(s // 4, s % 4) for s in slots}
    for p in range(6):
        for t in range(4):
            if (p, t) not in touched:
                assert (out[p, :, t] == pages[p, :, t]).all() and (osc[p, :, t] == scales[p, :, t]).all()


def test_planted_mistakes_fail():
    def ties_away(y):
        vals = fp8.e4m3_decode(FIN)
        pos = np.sort(np.unique(vals[vals >= 0]))
        a = np.abs(y)
        i = np.minimum(np.searchsorted(pos, a), len(pos) - 1)
        lo = np.maximum(i - 1, 0)
        pick = np.where(pos[i] - a <= a - pos[lo], pos[i], pos[lo])  # ties upward
        return np.sign(y) * pick
    pos = np.sort(np.unique(fp8.e4m3_decode(FIN)))
    pos = pos[pos > 0]
    mid = (pos[:-1] + pos[1:]) / 2
    assert not np.array_equal(ties_away(mid), fp8.e4m3_decode(fp8.e4m3_encode(mid)))

    x = np.random.default_rng(4).standard_normal((8, 256)).astype(np.float32)
    sc240 = (np.abs(x).reshape(8, 4, 64).max(-1) / np.float32(240)).astype(np.float16)
    y = np.clip(x.reshape(8, 4, 64) / sc240.astype(np.float32)[..., None], -448, 448)
    cmax = (fp8.e4m3_encode(y) & 0x7F).max(-1)
    assert not (cmax == 0x7E).all()
