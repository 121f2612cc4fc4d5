"""Shared helpers of the GPU parity tests (inputs from the generator, the
reference from the oracle, the result from the C ABI)."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from long_context_gqa_amd import binding as B
from long_context_gqa_amd import workloads as W
from oracle import attention as oatt

# the target tolerance: max |err| <= 2e-3 on outputs of order one (fp32 accumulation)
ATOL = 2e-3
# self-imposed: the same bound relative to the largest reference value, so the
# gate is not vacuous when outputs are far below one (literal-variant data)
RTOL_OF_MAX = 2e-3
LSE_ATOL = 1e-3


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def case(batch=1, q_len=8, lens=(100,), page_size=16, variant="unit", seed=7, order="per_request",
         kv_dtype="fp16", Hq=24, Hkv=4, device="cuda", bias=False, spare=None):
    wl = W.Workload("test", batch, q_len, ("fixed", 0), page_size, kv_dtype=kv_dtype, page_order=order,
                    bias_keys=bias, seed=seed, num_q_heads=Hq, num_kv_heads=Hkv)
    kv = [int(n) for n in lens]
    assert len(kv) == batch
    return W.make_verify_inputs(wl, variant, device=device, kv_lens=kv, spare_pages=spare)


def run_gpu(x: W.VerifyInputs, num_splits=0, max_kv_len=None, kv_lens=None, page_table=None, claim=False):
    dev = x.q.device
    kvl = (kv_lens if kv_lens is not None else x.kv_lens).to(dev)
    pt = (page_table if page_table is not None else x.page_table).to(dev).contiguous()
    mk = max_kv_len if max_kv_len is not None else int(kvl.max())
    out, lse, flags = B.verify_attention(x.q, x.k_pages, x.v_pages, pt, kvl, x.wl.q_len, mk,
                                         x.k_scales, x.v_scales, x.sm_scale, num_splits, claim=claim)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), int(flags.item())


def host(x: W.VerifyInputs):
    c = lambda t: None if t is None else t.cpu()
    return dict(q=c(x.q), k_pages=c(x.k_pages), v_pages=c(x.v_pages), k_scales=c(x.k_scales),
                v_scales=c(x.v_scales), page_table=x.page_table, kv_lens=x.kv_lens)


def oracle(x: W.VerifyInputs, groups=None, h=None):
    h = h or host(x)
    return oatt.verify_attention(h["q"], h["k_pages"], h["v_pages"], h["page_table"], h["kv_lens"],
                                 x.wl.q_len, x.sm_scale, h["k_scales"], h["v_scales"], rows=groups)


def rows_of(x: W.VerifyInputs, groups):
    """Boolean mask [B*q, Hq] of the (row, head) pairs covered by (b, g) groups."""
    q, G = x.wl.q_len, x.wl.num_q_heads // x.wl.num_kv_heads
    m = np.zeros((x.wl.batch * q, x.wl.num_q_heads), dtype=bool)
    for b, g in groups:
        m[b * q:(b + 1) * q, g * G:(g + 1) * G] = True
    return m


def check(out, lse, ref, ref_lse, mask=None, atol=ATOL, rtol_of_max=RTOL_OF_MAX, what=""):
    if mask is None:
        mask = ~np.isnan(ref_lse)
    o, r = out[mask], ref[mask]
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o - r).max() if o.size else 0.0
    scale = np.abs(r).max() if r.size else 1.0
    lerr = np.abs(lse[mask] - ref_lse[mask]).max() if o.size else 0.0
    # the same error in units of the output's own precision, on the large
    # outputs (|ref| >= max|ref| / 8, where the fp16 rounding of the output
    # eats most of the absolute gate): distance to the fp16 rounding of the
    # reference in fp16 ulps (0 or 1 for an exact kernel), and how far the
    # error goes past that rounding's half ulp
    ulps, past = 0.0, 0.0
    if o.size:
        big = np.abs(r) >= scale / 8
        r16 = r[big].astype(np.float16)
        ulp = np.spacing(np.abs(r16)).astype(np.float64)
        ulps = float((np.abs(o[big].astype(np.float64) - r16.astype(np.float64)) / ulp).max())
        past = float(np.maximum(np.abs(o[big] - r[big]) - 0.5 * ulp, 0.0).max())
    say(f"  {what}: max|err| {err:.3e}  max|ref| {scale:.3e}  rel {err / max(scale, 1e-30):.3e}  lse err {lerr:.3e}"
        f"  large outputs: fp16 ulps vs fp16(ref) {ulps:.0f}, beyond half an ulp {past:.2e}")
    assert err <= atol, f"{what}: max|err| {err} > {atol}"
    assert err <= rtol_of_max * scale, f"{what}: max|err| {err} > {rtol_of_max} * max|ref| {scale}"
    assert lerr <= LSE_ATOL, f"{what}: lse err {lerr}"
    return err
