"""Benchmark of the target-verify hot path on one MI355X.

One step = one verify of a block: paged causal GQA over the long cache
(sv_verify_attention: the split attention kernel plus the partial merge) and
greedy acceptance over the block's fp32 logits (sv_greedy_accept), on seeded
synthetic inputs already resident in HBM.

    python bench.py [--steps K] [--warmup W] [--config 3] [--variant literal] [--ragged] [--stochastic] [--topk]
                    [--window W --sink S] [--extend 64,256]

Prints one JSON line. `value` is the effective HBM bandwidth of the whole step
(algorithmic bytes of attention + accept / step time). The `roofline` object
is for the dominant kernel (verify_attn): its algorithmic bytes per launch
over its average launch duration, measured here with HIP events on the stream
the kernels run on (the attention call minus the merge kernel, timed
separately). `cpu_baseline` is the float64 oracle timed on the host on the
same workload's (request, KV head) groups, in order, for up to about 10 s
(the whole 512K workload takes about 3 s).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify-attn effective HBM GB/s (% of peak) at q=8, 512K ctx; verified tok/s"
PEAK_HBM_GBS = 8000.0
PEAK_MFMA_FP16_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--variant", default="literal", choices=["literal", "unit"])
    ap.add_argument("--splits", type=int, default=0, help="force the number of key chunks (0 = planner)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep-splits", default=None,
                    help="comma-separated split counts: time the verify attention call at each")
    ap.add_argument("--q-sweep", default=None,
                    help="comma list of q_len: the same K/V (same bytes) verified with that many rows per request")
    ap.add_argument("--cold", action="store_true",
                    help="also time the attention call after writing 1 GiB (evicting L2 and the Infinity Cache)")
    ap.add_argument("--reference-copy-mib", type=int, default=0,
                    help="time a device-to-device copy of this size as an attainable-bandwidth reference")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run a plain device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--ragged", action="store_true",
                    help="also time one round of blocks of a seeded width per request (2..q_len): block "
                         "preparation, K/V append, ragged verify attention and ragged greedy accept")
    ap.add_argument("--stochastic", action="store_true",
                    help="also time stochastic acceptance (rejection sampling) on the workload's logits with "
                         "seeded draft distributions")
    ap.add_argument("--topk", action="store_true",
                    help="also time top-16 candidate selection over the workload's logits")
    ap.add_argument("--window", type=int, default=0,
                    help="also time the sink + sliding-window verify with this window (positions)")
    ap.add_argument("--sink", type=int, default=0, help="leading sink positions for --window")
    ap.add_argument("--extend", default=None,
                    help="also time extend chunks of these widths (comma list, up to 512 rows per request) "
                         "over the workload's cache, against the fp16 MFMA peak")
    ap.add_argument("--claim", action="store_true",
                    help="also time the opt-in claimed-work mode (SV_VERIFY_CLAIMED_WORK; reproducible to rounding "
                         "only) against the default plan, alternating the two")
    ap.add_argument("--traffic", default=None,
                    help="JSON with measured HBM bytes per verify_attn launch (default: the one under "
                         "profiles/ for this workload, used only while the kernel source is unchanged)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "the verify path runs and is measured on one GPU (one MI355X); "
                                   "run with --gpus 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    from long_context_gqa_amd import binding as B
    from long_context_gqa_amd import workloads as W

    B.lib()  # fail loudly if libsv.so is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration_mib:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give
        # the scale between counter units and bytes moved
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] calibration copy of {args.copy_calibration_mib} MiB done")
    wl = W.WORKLOADS[args.config]
    log(f"[bench] workload {wl.name} ({args.variant}): generating inputs on the GPU")
    t0 = time.time()
    x = W.make_verify_inputs(wl, args.variant, device=dev)
    acc_in = W.make_accept_inputs(wl, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f} s; pool {tuple(x.k_pages.shape)} {x.k_pages.dtype}")

    kv_lens = x.kv_lens.to(dev)
    page_table = x.page_table.to(dev).contiguous()
    call = B.VerifyCall(x.q, x.k_pages, x.v_pages, page_table, kv_lens, wl.q_len, x.max_kv_len,
                        x.k_scales, x.v_scales, x.sm_scale, args.splits)
    acall = B.AcceptCall(acc_in.logits, acc_in.draft_ids, wl.q_len, kv_lens)
    stream = torch.cuda.current_stream()

    def step():
        call.run(stream)
        acall.run(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    flags = int(call.flags.item())
    if flags:
        raise SystemExit(f"kernel flagged a contract violation: {flags}")
    # sanity of the accept result against the planted lengths (the oracle's
    # job is in the tests; here only the generator's construction is used)
    if not torch.equal(acall.accept_len.cpu(), acc_in.planted_accept):
        raise SystemExit("accept lengths differ from the planted ones")

    # ---- timed region: K whole steps ------------------------------------
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = e0.elapsed_time(e1) / args.steps

    # ---- per-part timing (same stream, events around each launch) ---------
    def timed(fn, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs]) * 1e3  # us

    n_part = max(10, args.steps)
    attn_us = timed(lambda: call.run(stream), n_part)
    acc_us = timed(lambda: acall.run(stream), n_part)
    merge_us = np.zeros(1)
    if call.splits > 1:
        S, R, Hq, D = call.splits, x.q.shape[0], x.q.shape[1], x.q.shape[2]
        po_bytes = S * R * Hq * D * 4
        # the workspace: a block of work counters, then the partials (O, then lse)
        a256 = lambda n: (n + 255) // 256 * 256
        base = call.workspace.numel() - a256(po_bytes) - a256(S * R * Hq * 4)
        po = call.workspace[base:base + po_bytes].view(torch.float32).view(S, R, Hq, D)
        off = base + a256(po_bytes)
        pl = call.workspace[off:off + S * R * Hq * 4].view(torch.float32).view(S, R, Hq)
        mout = torch.empty_like(x.q)
        merge_us = timed(lambda: B.sv_verify_merge(po, pl, mout, None, stream), n_part)
    kern_us = float(np.median(attn_us) - np.median(merge_us))

    # ---- bytes ----------------------------------------------------------
    attn_bytes = W.verify_algorithmic_bytes(x.kv_lens.tolist(), wl.q_len, wl.num_q_heads, wl.num_kv_heads,
                                            wl.head_dim, wl.page_size, wl.kv_dtype)
    acc_bytes = W.accept_algorithmic_bytes(wl.batch, wl.q_len, wl.vocab)
    step_s = step_ms * 1e-3
    value = (attn_bytes + acc_bytes) / step_s / 1e9
    attn_gbs = attn_bytes / (np.median(attn_us) * 1e-6) / 1e9
    kern_gbs = attn_bytes / (kern_us * 1e-6) / 1e9
    rows = wl.batch * wl.q_len

    kernel = "verify_rows_kernel" if call.kernel == B.SV_KERNEL_TWO_HALVES else "verify_attn_kernel"
    traffic = measured_traffic(args.traffic, wl.name, kernel)

    sweep = None
    if args.sweep_splits:
        sweep = {}
        for sp in [int(v) for v in args.sweep_splits.split(",")]:
            c2 = B.VerifyCall(x.q, x.k_pages, x.v_pages, page_table, kv_lens, wl.q_len, x.max_kv_len,
                              x.k_scales, x.v_scales, x.sm_scale, sp)
            for _ in range(3):
                c2.run(stream)
            us = float(np.median(timed(lambda: c2.run(stream), n_part)))
            sweep[str(c2.splits)] = {"us": round(us, 2), "chunk": c2.chunk,
                                     "GBps": round(attn_bytes / (us * 1e-6) / 1e9, 1)}
            log(f"[bench] splits {c2.splits:4d} chunk {c2.chunk:6d}: {us:8.2f} us  "
                f"{attn_bytes / (us * 1e-6) / 1e9:8.1f} GB/s")
            del c2

    qsw = None
    if args.q_sweep:
        # fixed bytes: the same cache and lengths, q rows per request taken
        # from the workload's first verify row of each request
        qsw = {}
        q4 = x.q.view(wl.batch, wl.q_len, wl.num_q_heads, wl.head_dim)
        for qq in [int(v) for v in args.q_sweep.split(",")]:
            qx = q4[:, :1].repeat(1, qq, 1, 1).reshape(wl.batch * qq, wl.num_q_heads, wl.head_dim).contiguous()
            c2 = B.VerifyCall(qx, x.k_pages, x.v_pages, page_table, kv_lens, qq, x.max_kv_len,
                              x.k_scales, x.v_scales, x.sm_scale, 0)
            for _ in range(3):
                c2.run(stream)
            us = float(np.median(timed(lambda: c2.run(stream), n_part)))
            qb = W.verify_algorithmic_bytes(x.kv_lens.tolist(), qq, wl.num_q_heads, wl.num_kv_heads,
                                            wl.head_dim, wl.page_size, wl.kv_dtype)
            qsw[str(qq)] = {"us": round(us, 2), "splits": c2.splits, "GBps": round(qb / (us * 1e-6) / 1e9, 1)}
            log(f"[bench] q_len {qq:2d}: {us:8.2f} us  {qb / (us * 1e-6) / 1e9:8.1f} GB/s")
            del c2, qx

    cold = None
    if args.cold:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_part)]
        for i, (a, b) in enumerate(evs):
            flush.fill_(i & 0xFF)
            a.record(stream)
            call.run(stream)
            b.record(stream)
        torch.cuda.synchronize()
        cus = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
        cold = {"us_median": round(float(np.median(cus)), 2),
                "effective_GBps": round(attn_bytes / (np.median(cus) * 1e-6) / 1e9, 1),
                "note": "1 GiB written before each call; warm figures above"}
        del flush

    ref_copy = None
    if args.reference_copy_mib:
        n = args.reference_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        us = float(np.median(timed(lambda: dst.copy_(src), 20)))
        ref_copy = {"bytes_moved": 2 * n, "us": round(us, 2), "GBps": round(2 * n / (us * 1e-6) / 1e9, 1),
                    "note": "device copy (read + write) as an attainable-bandwidth reference"}
        del src, dst

    claimed = None
    if args.claim:
        cc = B.VerifyCall(x.q, x.k_pages, x.v_pages, page_table, kv_lens, wl.q_len, x.max_kv_len, x.k_scales,
                          x.v_scales, x.sm_scale, args.splits, claim=True)
        for _ in range(3):
            cc.run(stream)
        # alternate the two modes in rounds, so that drift over the run hits both alike
        us_c, us_d = [], []
        for _ in range(5):
            us_c.append(timed(lambda: cc.run(stream), n_part))
            us_d.append(timed(lambda: call.run(stream), n_part))
        uc, ud = float(np.median(np.concatenate(us_c))), float(np.median(np.concatenate(us_d)))
        claimed = {"us_median": round(uc, 2), "GBps": round(attn_bytes / (uc * 1e-6) / 1e9, 1),
                   "default_us_median": round(ud, 2), "default_GBps": round(attn_bytes / (ud * 1e-6) / 1e9, 1),
                   "splits": cc.splits, "flags": int(cc.flags.item())}
        log(f"[bench] claimed work {uc:.2f} us vs default {ud:.2f} us")
        del cc

    ragged = None
    if args.ragged:
        ragged = ragged_round(x, wl, acc_in, page_table, stream, timed, n_part)

    stoch = None
    if args.stochastic:
        si = W.make_sampling_inputs(wl, device=dev)
        rc = B.RejectionAcceptCall(acc_in.logits, si.draft_ids, si.draft_probs, wl.q_len, 1.0, si.u_accept,
                                   si.u_final, kv_lens)
        for _ in range(3):
            rc.run(stream)
        us = float(np.median(timed(lambda: rc.run(stream), n_part)))
        sb = W.rejection_accept_bytes(wl.batch, wl.q_len, wl.vocab)
        stoch = {"us_median": round(us, 2), "algorithmic_bytes": sb, "GBps": round(sb / (us * 1e-6) / 1e9, 1),
                 "accept_len": rc.accept_len.cpu().tolist()[:8], "temperature": 1.0}
        log(f"[bench] rejection accept: {us:.2f} us, {sb / (us * 1e-6) / 1e9:.1f} GB/s")
        del si, rc

    topk = None
    if args.topk:
        tc = B.TopkCall(acc_in.logits, 16)
        for _ in range(3):
            tc.run(stream)
        us = float(np.median(timed(lambda: tc.run(stream), n_part)))
        rows_k = acc_in.logits.shape[0]
        tb = rows_k * wl.vocab * 4 + rows_k * 16 * 8
        topk = {"rows": rows_k, "k": 16, "us_median": round(us, 2), "algorithmic_bytes": tb,
                "GBps": round(tb / (us * 1e-6) / 1e9, 1)}
        log(f"[bench] top-16 over {rows_k} rows: {us:.2f} us, {tb / (us * 1e-6) / 1e9:.1f} GB/s")
        del tc

    win = None
    if args.window > 0:
        wc = B.VerifyCall(x.q, x.k_pages, x.v_pages, page_table, kv_lens, wl.q_len, x.max_kv_len, x.k_scales,
                          x.v_scales, x.sm_scale, 0, window=args.window, sink=args.sink)
        for _ in range(3):
            wc.run(stream)
        us = float(np.median(timed(lambda: wc.run(stream), n_part)))
        # keys the block can see: [0, sink) and [L + 1 - window, kv) per request
        vis = []
        for n in x.kv_lens.tolist():
            lo = max(n - wl.q_len + 1 - args.window, 0)
            vis.append(min(args.sink, lo) + (n - lo))
        wb = W.verify_algorithmic_bytes(vis, wl.q_len, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size,
                                        wl.kv_dtype)
        win = {"window": args.window, "sink": args.sink, "us_median": round(us, 2), "visible_keys": sum(vis),
               "algorithmic_bytes": wb, "GBps": round(wb / (us * 1e-6) / 1e9, 1), "splits": wc.splits,
               "chunk_tokens": wc.chunk, "flags": int(wc.flags.item())}
        log(f"[bench] window {args.window} sink {args.sink}: {us:.2f} us over {sum(vis)} visible keys")
        del wc

    ext = None
    if args.extend:
        ext = []
        for qe in [int(v) for v in args.extend.split(",")]:
            # an extend chunk of qe new tokens: the last qe positions of each
            # request's cache, with query rows of the generator's scale
            gen = torch.Generator(device=dev).manual_seed(1000 + qe)
            qx = (torch.randn((wl.batch * qe, wl.num_q_heads, wl.head_dim), generator=gen, device=dev)
                  ).to(torch.float16)
            ec = B.VerifyCall(qx, x.k_pages, x.v_pages, page_table, kv_lens, qe, x.max_kv_len, x.k_scales,
                              x.v_scales, x.sm_scale, 0)
            for _ in range(3):
                ec.run(stream)
            us = float(np.median(timed(lambda: ec.run(stream), n_part)))
            # QK^T and PV: 2 * 2 * D flops per (row, head, visible key)
            keys = sum(qe * (n - qe) + qe * (qe + 1) // 2 for n in x.kv_lens.tolist())
            flops = 4 * wl.head_dim * wl.num_q_heads * keys
            eb = W.verify_algorithmic_bytes(x.kv_lens.tolist(), qe, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                            wl.page_size, wl.kv_dtype)
            tf = flops / (us * 1e-6) / 1e12
            ext.append({"q_len": qe, "us_median": round(us, 2), "flops": flops, "TFLOPs": round(tf, 1),
                        "frac_mfma_fp16": round(tf / PEAK_MFMA_FP16_TFLOPS, 4), "algorithmic_bytes": eb,
                        "GBps": round(eb / (us * 1e-6) / 1e9, 1), "splits": ec.splits, "chunk_tokens": ec.chunk,
                        "flags": int(ec.flags.item())})
            log(f"[bench] extend {qe}: {us:.2f} us, {tf:.1f} TFLOP/s ({100 * tf / PEAK_MFMA_FP16_TFLOPS:.1f}% of "
                f"fp16 MFMA), {eb / (us * 1e-6) / 1e9:.1f} GB/s, splits {ec.splits}")
            del ec, qx

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x, wl)

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if wl.kv_dtype == "fp16" else "e4m3",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": wl.batch, "q_len": wl.q_len, "max_kv_len": x.max_kv_len,
            "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
            "page_size": wl.page_size, "kv_dtype": wl.kv_dtype, "variant": args.variant,
            "splits": call.splits, "chunk_tokens": call.chunk,
        },
        "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
        "verify_attention": {
            "us_median": round(float(np.median(attn_us)), 2),
            "us_p10": round(float(np.percentile(attn_us, 10)), 2),
            "us_p90": round(float(np.percentile(attn_us, 90)), 2),
            "effective_GBps": round(attn_gbs, 1),
            "pct_of_peak_hbm": round(100 * attn_gbs / PEAK_HBM_GBS, 2),
            "verified_tok_per_s": round(rows / (np.median(attn_us) * 1e-6), 1),
            "algorithmic_bytes": attn_bytes,
            "merge_us_median": round(float(np.median(merge_us)), 2),
        },
        "greedy_accept": {
            "us_median": round(float(np.median(acc_us)), 2),
            "effective_GBps": round(acc_bytes / (np.median(acc_us) * 1e-6) / 1e9, 1),
            "algorithmic_bytes": acc_bytes,
        },
        "roofline": {
            "kernel": kernel,
            "bound": "hbm",
            "achieved": round(kern_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(kern_gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "launch_us": round(kern_us, 2),
            "bytes_per_launch": attn_bytes,
        },
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
        "split_sweep": sweep,
        "q_sweep": qsw,
        "verify_attention_cold": cold,
        "reference_copy": ref_copy,
        "verify_attention_claimed": claimed,
        "ragged_round": ragged,
        "rejection_accept": stoch,
        "topk_candidates": topk,
        "window_verify": win,
        "extend_chunks": ext,
    }
    print(json.dumps(res), flush=True)


def ragged_round(x, wl, acc_in, page_table, stream, timed, n):
    """One verify round with a seeded width per request (2..q_len), on the
    workload's cache: prepare_block, the K/V append (rewriting the block rows
    with the values already there; an FP8 cache gets them dequantised and
    quantised again), ragged verify attention and ragged greedy accept, each
    timed alone."""
    import numpy as np
    import torch

    from long_context_gqa_amd import binding as B
    from long_context_gqa_amd import workloads as W
    dev = x.q.device
    q = wl.q_len
    widths = W.block_widths(wl, lo=min(2, q))
    prefixes = [int(k) - q for k in x.kv_lens.tolist()]
    rows = sum(widths)
    i32 = dict(dtype=torch.int32, device=dev)
    seq = torch.tensor(prefixes, **i32)
    last = torch.zeros(wl.batch, **i32)  # t0 of each block (never compared)
    prep = B.PrepareCall(seq, torch.tensor(widths, **i32), page_table, q, wl.page_size, x.num_pages,
                         last, acc_in.draft_ids if q > 1 else None)
    prep.run(stream)
    torch.cuda.synchronize()
    if prep.flags.item() or prep.q_start[-1].item() != rows:
        raise SystemExit("block preparation flagged or miscounted the rows")
    res = {"widths": widths, "rows": rows, "batch": wl.batch, "max_width": q}
    res["prepare_us"] = round(float(np.median(timed(lambda: prep.run(stream), n))), 2)

    P = wl.page_size
    sl = prep.cache_slot[:rows].long()
    if wl.kv_dtype == "fp16":
        nk = x.k_pages[sl // P, :, sl % P].contiguous()
        nv = x.v_pages[sl // P, :, sl % P].contiguous()
        ab = 2 * 2 * nk.numel() * 2 + rows * 4  # K and V rows read and written, slots read

        def app():
            B.sv_append_kv(nk, nv, prep.cache_slot, prep.q_start, wl.batch, wl.batch * q, x.k_pages, x.v_pages,
                           prep.flags, stream)
    else:
        # the rows' dequantised values, quantised again into their slots
        def deq(pages, scales):
            codes = pages[sl // P, :, sl % P].contiguous().view(torch.float8_e4m3fn).to(torch.float32)
            return (codes * scales[sl // P, :, sl % P].float().repeat_interleave(64, -1)).to(torch.float16)
        nk, nv = deq(x.k_pages, x.k_scales), deq(x.v_pages, x.v_scales)
        # fp16 rows read; E4M3 codes and fp16 scales written; slots read
        ab = 2 * (nk.numel() * 2 + nk.numel() + nk.numel() // 64 * 2) + rows * 4

        def app():
            B.sv_append_kv_fp8(nk, nv, prep.cache_slot, prep.q_start, wl.batch, wl.batch * q, x.k_pages, x.v_pages,
                               x.k_scales, x.v_scales, prep.flags, stream)
    app()
    us = float(np.median(timed(app, n)))
    res.update(append_us=round(us, 2), append_GBps=round(ab / (us * 1e-6) / 1e9, 1), append_bytes=ab)

    qp = W.pack_rows(x.q, q, widths)
    rc = B.RaggedVerifyCall(qp, prep.q_start, x.k_pages, x.v_pages, page_table, prep.kv_lens_out, q, x.max_kv_len,
                            x.k_scales, x.v_scales, x.sm_scale, 0)
    for _ in range(3):
        rc.run(stream)
    us = float(np.median(timed(lambda: rc.run(stream), n)))
    if rc.flags.item():
        raise SystemExit(f"ragged verify flagged a contract violation: {rc.flags.item()}")
    vb = W.verify_algorithmic_bytes([p_ + w for p_, w in zip(prefixes, widths)], widths, wl.num_q_heads,
                                    wl.num_kv_heads, wl.head_dim, wl.page_size, wl.kv_dtype)
    gbs = vb / (us * 1e-6) / 1e9
    res.update(verify_us=round(us, 2), verify_GBps=round(gbs, 1), verify_pct_of_peak_hbm=round(100 * gbs / 8000, 2),
               verified_tok_per_s=round(rows / (us * 1e-6), 1), verify_algorithmic_bytes=vb,
               splits=rc.splits, chunk_tokens=rc.chunk)

    logits = W.pack_rows(acc_in.logits, q, widths)
    ac = B.RaggedAcceptCall(logits, prep.block_ids, prep.q_start, wl.batch, q, prep.kv_lens_out)
    ac.run(stream)
    us = float(np.median(timed(lambda: ac.run(stream), n)))
    # planted lengths cut at each width (the drafts before the cut are the same)
    expect = torch.minimum(acc_in.planted_accept, torch.tensor(widths, dtype=torch.int32) - 1)
    if not torch.equal(ac.accept_len.cpu(), expect):
        raise SystemExit("ragged accept lengths differ from the planted ones cut at each width")
    accb = rows * wl.vocab * 4 + rows * 4 + (wl.batch + 1) * 4 + 3 * wl.batch * 4
    res.update(accept_us=round(us, 2), accept_GBps=round(accb / (us * 1e-6) / 1e9, 1), accept_bytes=accb)
    log(f"[bench] ragged round: {rows} rows; prepare {res['prepare_us']} us, append {res.get('append_us')} us, "
        f"verify {res['verify_us']} us ({res['verify_GBps']} GB/s), accept {res['accept_us']} us")
    return res


def measured_traffic(path, workload, kernel):
    """HBM bytes (FETCH + WRITE) per launch of the attention kernel from the
    rocprofv3 counter runs recorded under profiles/, or None when there is no
    record for this workload and kernel or the kernel's source has changed
    since it was taken."""
    import hashlib
    path = path or os.path.join(ROOT, "profiles", f"traffic_verify_attn_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel", "verify_attn_kernel") != kernel:
        return None
    # the kernel's source files, hashed in the listed order as one byte string
    h = hashlib.sha256()
    for src in rec.get("sources") or [rec["source"]]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]


def cpu_baseline(x, wl, budget_s=10.0):
    """The float64 oracle on (request, KV head) groups of the workload, in
    order, until about budget_s seconds of oracle time have been spent or the
    workload is done: all q_len x G rows of each group over its request's
    whole cache. Reported in the metric's unit (the groups' algorithmic bytes
    over the oracle's wall time)."""
    import numpy as np

    from long_context_gqa_amd import workloads as W
    from oracle import attention as oatt
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count()
    G = wl.num_q_heads // wl.num_kv_heads
    spent, done, sample_bytes, keys = 0.0, 0, 0, 0
    for b in range(wl.batch):
        n = int(x.kv_lens[b])
        npg = (n + wl.page_size - 1) // wl.page_size
        ids = x.page_table[b, :npg].long().to(x.k_pages.device)
        # hand the oracle a compact pool holding this request's pages only
        kp = x.k_pages[ids].cpu()
        vp = x.v_pages[ids].cpu()
        ks = x.k_scales[ids].cpu() if x.k_scales is not None else None
        vs = x.v_scales[ids].cpu() if x.v_scales is not None else None
        table = np.arange(npg, dtype=np.int32)[None]
        q = x.q[b * wl.q_len:(b + 1) * wl.q_len].cpu()
        for g in range(wl.num_kv_heads):
            log(f"[bench] cpu baseline: oracle on request {b}, KV head {g} ({n} keys)")
            t0 = time.perf_counter()
            oatt.verify_attention(q, kp, vp, table, np.array([n]), wl.q_len, x.sm_scale, ks, vs, rows=[(0, g)])
            spent += time.perf_counter() - t0
            done += 1
            keys += n
            sample_bytes += n * W.kv_bytes_per_token_head(wl.head_dim, wl.kv_dtype) + 2 * wl.q_len * G * wl.head_dim * 2
            if spent >= budget_s:
                break
        del kp, vp, ks, vs
        if spent >= budget_s:
            break
    total = wl.batch * wl.num_kv_heads
    what = "the whole workload" if done == total else f"the first {done} of {total}"
    return {
        "value": round(sample_bytes / spent / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"float64 oracle on {what} (request, KV head) groups: {wl.q_len}x{G} rows each, {keys} keys in "
                  f"all ({sample_bytes} algorithmic bytes) in {spent:.2f} s; host has {os.cpu_count()} CPUs, "
                  f"{len(os.sched_getaffinity(0))} usable by this process",
        "seconds": round(spent, 2),
    }


if __name__ == "__main__":
    main()
