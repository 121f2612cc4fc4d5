"""GPU parity of the verify attention's dispatch over whole batches against
the float64 oracle. Batches of 2..64 requests take the longest-first order
(full chunks in split-major order, then the last partial chunks, longest
first); larger batches keep the split-major numbering. Both orders must give
every request exactly its own chunks: ragged lengths, zero widths, a request
with rows but no visible key, forced and automatic splits, one and two row
tiles, fp16 and FP8."""
import numpy as np
import pytest
import torch

from helpers import case, check, host, run_gpu, say
from oracle import attention as oatt
from test_gpu_block import ragged_case, ragged_oracle, run_ragged

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("Bn,kv_dtype,splits", [(2, "fp16", 0), (17, "fp16", 3), (64, "fp8_e4m3", 0),
                                                 (64, "fp16", 5), (70, "fp16", 0)])
def test_ragged_batches_every_request_gets_its_chunks(Bn, kv_dtype, splits):
    rng = np.random.default_rng(Bn * 10 + splits)
    widths = [int(w) for w in rng.integers(0, 9, Bn)]
    widths[0] = 8
    prefixes = [int(p) for p in rng.choice([0, 1, 15, 16, 17, 300, 1500, 3000], Bn)]
    x, q, kv, qs, qmax = ragged_case(widths, prefixes, 16, kv_dtype, seed=Bn + 3)
    say(f"B={Bn} {kv_dtype} splits={splits}: widths {widths[:12]}..., prefixes {prefixes[:12]}...")
    out, lse, flags = run_ragged(x, q, kv, qs, qmax, splits)
    assert flags == 0
    ref, ref_lse = ragged_oracle(x, q, kv, qs, widths)
    check(out, lse, ref, ref_lse, what=f"B={Bn}")


@pytest.mark.parametrize("Bn,q_len,Hq", [(40, 8, 24), (9, 16, 24), (66, 4, 24)])
def test_uniform_batches_with_ragged_lengths(Bn, q_len, Hq):
    # q_len 16 at G = 6: 96 rows per KV head, two row tiles per unit
    rng = np.random.default_rng(Bn + q_len)
    lens = [int(n) for n in rng.integers(q_len, 2500, Bn)]
    x = case(Bn, q_len, lens, 16, Hq=Hq, seed=Bn)
    out, lse, flags = run_gpu(x)
    assert flags == 0
    h = host(x)
    ref, ref_lse = oatt.verify_attention(h["q"], h["k_pages"], h["v_pages"], h["page_table"], h["kv_lens"], q_len,
                                         x.sm_scale)
    check(out, lse, ref, ref_lse, what=f"B={Bn} q={q_len}")


def test_request_with_rows_but_no_visible_key():
    # kv_len 0 for request 2 (below its block): its rows get 0 and -inf and
    # the flag; every other request matches the oracle
    lens = [600, 900, 300, 50, 1200, 16, 777]
    x = case(len(lens), 8, lens, 16, seed=5)
    kv = x.kv_lens.clone()
    kv[2] = 0
    out, lse, flags = run_gpu(x, kv_lens=kv, max_kv_len=max(lens))
    assert flags & 2
    q = 8
    assert (out[2 * q:3 * q] == 0).all() and np.isneginf(lse[2 * q:3 * q]).all()
    h = host(x)
    keep = [b for b in range(len(lens)) if b != 2]
    groups = [(b, g) for b in keep for g in range(4)]
    ref, ref_lse = oatt.verify_attention(h["q"], h["k_pages"], h["v_pages"], h["page_table"], h["kv_lens"], q,
                                         x.sm_scale, rows=groups)
    rows = np.concatenate([np.arange(b * q, (b + 1) * q) for b in keep])
    check(out[rows], lse[rows], ref[rows], ref_lse[rows], what="other requests")
