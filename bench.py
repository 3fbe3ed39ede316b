#!/usr/bin/env python3
"""GQLA decode attention benchmark on one MI355X.

Workload: the flagship decode step, bf16, batch 128, h_q = 128 query heads in
g = 8 groups (16 heads per group), latent width r_kv = 512, rotary key width
d_R = 64, per-group head width d_h = 128, uniform context 8192, s_q = 1.
Synthetic seeded inputs (synth.inputs), resident in HBM before timing.

A step is one pass of the whole hot path over the batch: the MQA-absorb path
(query absorption, latent attention with split-K, log-sum-exp combine with
the fused W_UV up-projection) and the GQA path (attention over the expanded
group rows with split-K, combine).  The group rows are expanded once per
sequence beforehand (the method expands the latent once, not per step); that
expansion is timed on its own and reported as expand_ms.

Before the W warm-up steps the step is run until the GPU's clock has settled
(reported as "settle"): under this load MI355X's power management first drops the
SIMD clock to about 1.3 GHz a few launches in and then raises it again over the next
~50 launches (up to ~1.9 GHz), so a run that starts timing after a few steps
would measure that transient rather than the steady state.

Prints ONE JSON line: query-tokens/s of the step (batch * s_q / step time),
per-path times and roofline fractions, the roofline object of the dominant
kernel (HIP events around that kernel on its own stream) and the fp64 CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode query-tokens/s + % HBM/MFMA roofline, h_q=128 g=8 ctx 8K, both paths"
PEAK_HBM = 8.0e12          # MI355X HBM3E, bytes/s
PEAK_BF16 = 2.5e15         # MI355X dense bf16 MFMA, flop/s
COPY_BYTES = 1 << 30       # plain device copy run once per bench (counter calibration)


# name -> (config id, overrides, description).  The flagship is the metric's workload; the
# others are the remaining bf16 decode shapes, measured with the same step (both paths).
WORKLOADS = {
    "flagship": (3, {}, "gqla-decode-flagship: both paths, bf16, batch 128, h_q 128, g 8, r_kv 512, "
                        "d_R 64, d_h 128, ctx 8192 uniform, s_q 1"),
    "llama3-8b": (2, {}, "LLaMA-3-8B-derived shape: both paths, bf16, batch 64, h_q 32, g 8, ctx 4096 uniform, s_q 1"),
    "mtp-g8-sq2": (4, {"g": 8, "s_q": 2}, "multi-token step: both paths, bf16, batch 256, h_q 128, g 8, s_q 2, "
                                          "ctx ragged in [1024, 32768]"),
    "mtp-g4-sq1": (4, {"g": 4, "s_q": 1}, "multi-token shape at g 4: both paths, bf16, batch 256, h_q 128, g 4, "
                                          "s_q 1, ctx ragged in [1024, 32768]"),
    "long-context": (5, {}, "long context split-K: both paths, bf16, batch 16, h_q 128, g 8, s_q 1, "
                            "ctx ragged in [65536, 131072]"),
}


def note(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the CPU oracle baseline")
    ap.add_argument("--settle-min", type=int, default=120,
                    help="clock settling: at least this many steps before the warm-up (0: no settling)")
    ap.add_argument("--settle-max", type=int, default=600, help="clock settling: at most this many steps")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg (CPU baseline and its sampled agreement check)")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="flagship",
                    help="decode workload (default: the flagship step the metric is quoted on)")
    return ap.parse_args(argv)




def cpu_baseline(cfg, budget_s, gpu_out):
    """The fp64 oracle's plain definition (textbook_decode: per-group K and V materialised
    from the latent rows, then softmax attention) timed on sampled sequences.

    gpu_out maps path -> device output [B][s_q][h_q][d_h]; the sampled sequences are also
    compared with it (|gpu - oracle| / (2e-3 + 2e-2 |oracle|); the GQA output comes from
    rows the device expanded, whose bf16 rounding averages out at these lengths).
    """
    import numpy as np
    import oracle
    import synth
    from synth.inputs import sample_sequences
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    qn, qr = synth.queries(cfg)
    w_uk, w_uv = synth.up_weights(cfg)
    spent, n, worst = 0.0, 0, 0.0
    for b in sample_sequences(cfg, cfg.batch):
        L = synth.ctx_len(cfg, b)
        rows = synth.latent_rows(cfg, b, L)
        t0 = time.perf_counter()
        ref, _ = oracle.textbook_decode(rows, qn[b], qr[b], w_uk, w_uv, L, cfg.scale)
        spent += time.perf_counter() - t0
        n += 1
        for path in ("absorb", "gqa"):
            got = gpu_out[path][b].float().cpu().numpy().astype(np.float64)
            worst = max(worst, float(np.max(np.abs(got - ref) / (2e-3 + 2e-2 * np.abs(ref)))))
        if spent >= budget_s:
            break
    rec = {"value": round(n * cfg.s_q / spent, 3), "unit": "query-tokens/s", "cores": cores, "kind": "oracle",
           "sample": f"{n} of {cfg.batch} sequences at ctx {cfg.ctx[0]}: the fp64 numpy oracle's textbook form "
                     f"(K and V of every group materialised from the latent rows, then softmax attention), "
                     f"{spent:.1f} s on {cores} cores (BLAS threads {blas_threads})"}
    parity = {"sequences": n, "max_err_over_tol": round(worst, 4), "ok": worst <= 1.0}
    return rec, parity


def next_rows(gqla, rf, cfg, sh, w, gc, dev, warmup, steps):
    """The steps around the decode path, on the flagship batch (not part of the metric):
    sparse GQLA decode over 2048 listed rows per (sequence, group), the decode-step append
    of one new token per sequence (rows, rotary keys and queries, expanded rows), and the
    path the roofline selector picks from this device's measured peaks."""
    import torch
    B, S = cfg.batch, w.max_ctx
    out = {}

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for e in (k0, k1):
            e.record()
        torch.cuda.synchronize()
        kern, call = [], []
        for _ in range(steps):
            gqla.set_kernel_events(k0, k1)
            c0.record()
            fn()
            c1.record()
            gqla.set_kernel_events(None, None)
            torch.cuda.synchronize()
            kern.append(k0.elapsed_time(k1))
            call.append(c0.elapsed_time(c1))
        return sum(kern) / len(kern), sum(call) / len(call)

    topk = 2048
    gen = torch.Generator(device=dev).manual_seed(7)
    idx = torch.rand((B, cfg.s_q, cfg.g, S), device=dev, generator=gen).argsort(dim=-1)[..., :topk].to(torch.int32)
    idx = idx.contiguous()
    o = torch.empty((B, cfg.s_q, cfg.h_q, cfg.d_h), dtype=torch.bfloat16, device=dev)
    ws = gqla.alloc_workspace(sh, gqla.SPARSE, B, topk, 0, dev)
    kern, call = timed(lambda: gqla.decode_gqa_sparse(sh, w.q_nope, w.q_rope, gc, w.ctx_lens, idx, o, None, ws))
    # gathered K_j, V_j and k_R of every listed row, its index, queries in, outputs out
    alg = (B * cfg.s_q * cfg.g * topk * ((2 * cfg.d_h + cfg.d_r) * 2 + 4)
           + B * cfg.s_q * cfg.h_q * (cfg.d_h + cfg.d_r + cfg.d_h) * 2)
    out["sparse_gqa"] = {"topk": topk, "kernel": "gqa_sparse_kernel", "kernel_ms": round(kern, 4),
                         "call_ms": round(call, 4), "alg_bytes_per_launch": alg,
                         "hbm_frac": round(alg / (kern * 1e-3) / rf.MI355X.bw, 4),
                         "n_split": gqla.plan_splits(sh, gqla.SPARSE, B, topk, 0)[0]}
    del idx, ws

    g = torch.Generator(device=dev).manual_seed(8)
    c_new = torch.randn((B, cfg.s_q, cfg.r_kv), device=dev, generator=g).to(torch.bfloat16)
    kr = torch.randn((B, cfg.s_q, cfg.d_r), device=dev, generator=g).to(torch.bfloat16)
    qraw = torch.randn((B, cfg.s_q, cfg.h_q, cfg.d_r), device=dev, generator=g).to(torch.bfloat16)
    qrot = torch.empty_like(qraw)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)

    def append():
        gqla.append_rows(sh, c_new, kr, w.ctx_lens, w.latent, qraw, qrot, 10000.0, w.w_uk, w.w_uv, gc)
    for _ in range(warmup):
        append()
    t0.record()
    for _ in range(steps):
        append()
    t1.record()
    torch.cuda.synchronize()
    out["append"] = {"tokens": B * cfg.s_q, "ms": round(t0.elapsed_time(t1) / steps, 4), "with_group_rows": True}

    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    bw, fl = gqla.measure_peaks(scratch)
    del scratch
    sel = {}
    for max_sq in (1, 2):
        shp = gqla.make_shape(cfg.h_q, cfg.g, cfg.r_kv, cfg.d_r, cfg.d_h, max_sq, cfg.scale, gqla.BF16)
        ch = gqla.select_path(shp, B, int(w.lens.sum()), fl, bw)
        sel[f"max_s_q={max_sq}"] = {"path": "absorb" if ch.path == gqla.ABSORB else "gqa", "s_q": ch.s_q,
                                     "roofline_tokens_per_s": round(ch.tokens_per_s, 1),
                                     "compute_bound": bool(ch.compute_bound)}
    out["path_selector"] = {"measured_hbm_bytes_per_s": round(bw, 1), "measured_mfma_flops": round(fl, 1),
                            "measured_ridge": round(fl / bw, 1), "choice": sel}
    return out


def main(argv=None):
    args = parse(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the decode path runs on a single MI355X.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    from latent_kv_cache_amd import gqla
    from latent_kv_cache_amd import roofline as rf
    from bench_traffic import load_traffic
    from synth.device import make_workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gqla.load()
    cfg_id, overrides, workload_desc = WORKLOADS[args.workload]
    cfg = synth.config(cfg_id, **overrides)
    flagship = args.workload == "flagship"
    note(f"workload {args.workload}: generating inputs")
    t_gen = time.perf_counter()
    w = make_workload(cfg, device=dev)
    t_gen = time.perf_counter() - t_gen
    note(f"inputs ready in {t_gen:.1f} s; expanding group rows")
    B, S = cfg.batch, w.max_ctx
    total_ctx = int(w.lens.sum())
    sh = gqla.make_shape(cfg.h_q, cfg.g, cfg.r_kv, cfg.d_r, cfg.d_h, cfg.s_q, cfg.scale, gqla.BF16)

    # plain copy of known size: reference point for the HBM byte counters of profiled runs
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    del src, dst

    width = 2 * cfg.g * cfg.d_h + cfg.d_r
    gc = torch.empty((B, S, width), dtype=torch.bfloat16, device=dev)
    gqla.expand_groups(sh, w.latent, w.w_uk, w.w_uv, w.ctx_lens, gc)   # first touch of gc, untimed

    out_a = torch.empty((B, cfg.s_q, cfg.h_q, cfg.d_h), dtype=torch.bfloat16, device=dev)
    out_g = torch.empty_like(out_a)
    # split-K partition planned from the context lengths, which the host holds here
    ns_a = gqla.plan_splits_lens(sh, gqla.ABSORB, w.lens, S)[0]
    ns_g = gqla.plan_splits_lens(sh, gqla.GQA, w.lens, S)[0]
    ws_a = gqla.alloc_workspace(sh, gqla.ABSORB, B, S, ns_a, dev)
    ws_g = gqla.alloc_workspace(sh, gqla.GQA, B, S, ns_g, dev)
    split_a = gqla.plan_splits(sh, gqla.ABSORB, B, S, ns_a)
    split_g = gqla.plan_splits(sh, gqla.GQA, B, S, ns_g)

    def absorb():
        gqla.decode_absorb(sh, w.q_nope, w.q_rope, w.w_uk, w.w_uv, w.latent, w.ctx_lens, out_a, None, ws_a,
                           num_splits=ns_a)

    def gqa():
        gqla.decode_gqa(sh, w.q_nope, w.q_rope, gc, w.ctx_lens, out_g, None, ws_g, num_splits=ns_g)

    # clock settling: steps until the step time of the last 20 is within 1 % of the 20
    # before them (after at least settle_min steps)
    settle = {"steps": 0, "ms": 0.0, "first_step_ms": None, "last_step_ms": None}
    if args.settle_min > 0:
        note("settling clocks")
        sa, sb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        hist = []
        t_set = time.perf_counter()
        while True:
            sa.record()
            absorb()
            gqa()
            sb.record()
            sb.synchronize()
            hist.append(sa.elapsed_time(sb))
            n = len(hist)
            if n >= max(args.settle_min, 40):
                prev, last = float(np.mean(hist[-40:-20])), float(np.mean(hist[-20:]))
                if abs(last - prev) <= 0.01 * last:
                    break
            if n >= args.settle_max:
                break
        settle = {"steps": len(hist), "ms": round((time.perf_counter() - t_set) * 1e3, 1),
                  "first_step_ms": round(hist[0], 4), "last_step_ms": round(float(np.mean(hist[-20:])), 4)}

    note("warm-up")
    for _ in range(args.warmup):
        absorb()
        gqa()
    torch.cuda.synchronize()
    note("timed steps")

    K = args.steps
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    ev = {k: [mk() for _ in range(K)] for k in ("a0", "a1", "ak0", "ak1", "g0", "g1", "gk0", "gk1")}
    for lst in ev.values():        # materialise the events before the library records them
        for e in lst:
            e.record()
    torch.cuda.synchronize()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev["a0"][i].record()
        gqla.set_kernel_events(ev["ak0"][i], ev["ak1"][i])
        absorb()
        ev["a1"][i].record()
        ev["g0"][i].record()
        gqla.set_kernel_events(ev["gk0"][i], ev["gk1"][i])
        gqa()
        ev["g1"][i].record()
    gqla.set_kernel_events(None, None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K

    # the expansion (once per token, outside the metric), timed after the steps with the
    # clock settled: median of 10 calls
    ex = []
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gqla.expand_groups(sh, w.latent, w.w_uk, w.w_uv, w.ctx_lens, gc)
        e1.record()
        e1.synchronize()
        ex.append(e0.elapsed_time(e1))
    expand_ms = float(np.median(ex))

    def avg(a, b):
        return float(np.mean([ev[a][i].elapsed_time(ev[b][i]) for i in range(K)]))

    call_a, call_g = avg("a0", "a1"), avg("g0", "g1")
    kern_a, kern_g = avg("ak0", "ak1"), avg("gk0", "gk1")

    work_a = rf.step_work("absorb", cfg.h_q, cfg.g, cfg.s_q, total_ctx, B, cfg.r_kv, cfg.d_r, cfg.d_h)
    work_g = rf.step_work("gqa", cfg.h_q, cfg.g, cfg.s_q, total_ctx, B, cfg.r_kv, cfg.d_r, cfg.d_h)
    q_tokens = B * cfg.s_q

    def path_rec(work, call_ms, kern_ms, splits, kernel):
        t = call_ms * 1e-3
        hbm = work.bytes / t / PEAK_HBM
        mfma = work.flops / t / PEAK_BF16
        roof_t = max(work.bytes / PEAK_HBM, work.flops / PEAK_BF16)
        return {"ms": round(call_ms, 4), "tokens_per_s": round(q_tokens / t, 1),
                "hbm_frac": round(hbm, 4), "mfma_frac": round(mfma, 4),
                "roofline_frac": round(roof_t / t, 4),
                "roofline_tokens_per_s": round(q_tokens / roof_t, 1),
                "alg_bytes": work.bytes, "alg_flops": work.flops,
                "main_kernel": kernel, "main_kernel_ms": round(kern_ms, 4),
                "n_split": splits[0], "chunk": splits[1]}

    rq = cfg.s_q * cfg.h_q
    absorb_name = "absorb_decode_kernel<%d>" % min(4, rq // 16)
    # the GQA launcher's choice: two row tiles per wave when a group has an even number
    # of 16-row tiles and one per wave would need more than one workgroup; tiles loaded
    # straight into LDS (16 rows at g = 8, 32 below) except at g = 1 and, at g = 8 with
    # one row tile per wave, for chunks longer than 1024 tokens
    rt = (cfg.s_q * (cfg.h_q // cfg.g) + 15) // 16
    two = rt % 2 == 0 and cfg.g * rt > 8
    rpw = 2 if two else 1
    tr = 16 if cfg.g == 8 else 32
    if cfg.g == 1:
        gqa_name = "gqa_decode_kernel<1, 8, %d, %d>" % (rpw, 1 if two else 2)
    elif cfg.g == 8 and not two and split_g[1] > 1024:
        gqa_name = "gqa_decode_kernel<8, 8, 1, 1>"
    else:
        gqa_name = "gqa_dma_kernel<%d, 8, %d, %d>" % (cfg.g, rpw, tr)
    paths = {"absorb": path_rec(work_a, call_a, kern_a, split_a, absorb_name),
             "gqa": path_rec(work_g, call_g, kern_g, split_g, gqa_name)}

    # dominant kernel: the longer of the two main attention kernels; its binding roof is
    # the one its algorithmic bytes and flops per launch reach first
    def kernel_roofline(kernel, alg_bytes, alg_flops, avg_ms, traffic):
        t = avg_ms * 1e-3
        if alg_bytes / PEAK_HBM >= alg_flops / PEAK_BF16:
            achieved, peak, unit, bound = alg_bytes / t / 1e9, PEAK_HBM / 1e9, "GB/s", "hbm"
        else:
            achieved, peak, unit, bound = alg_flops / t / 1e12, PEAK_BF16 / 1e12, "TFLOP/s", "mfma"
        return {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": kernel,
                "alg_bytes_per_launch": alg_bytes, "alg_flops_per_launch": alg_flops, "avg_ms": round(avg_ms, 4)}

    if kern_g >= kern_a:
        # bytes per launch: expanded rows of every cached token, queries in, outputs out
        alg = (rf.gqa_bytes_per_token(cfg.g, cfg.d_h, cfg.d_r) * total_ctx
               + q_tokens * cfg.h_q * (cfg.d_h + cfg.d_r + cfg.d_h) * 2)
        flops = 2 * cfg.s_q * cfg.h_q * (2 * cfg.d_h + cfg.d_r) * total_ctx
        roof = kernel_roofline(gqa_name, alg, flops, kern_g, load_traffic("gqa_decode", workload_desc))
    else:
        # latent rows, absorbed queries in (bf16 equivalent), outputs out, W_UV; flops of the
        # scores and values per cached token plus the fused W_UV epilogue
        alg = (rf.absorb_bytes_per_token(cfg.r_kv, cfg.d_r) * total_ctx
               + q_tokens * cfg.h_q * (cfg.r_kv + cfg.d_r + cfg.d_h) * 2 + cfg.g * cfg.d_h * cfg.r_kv * 2)
        flops = (2 * cfg.s_q * cfg.h_q * (2 * cfg.r_kv + cfg.d_r) * total_ctx
                 + 2 * q_tokens * cfg.h_q * cfg.d_h * cfg.r_kv)
        roof = kernel_roofline(absorb_name, alg, flops, kern_a, load_traffic("absorb_decode", workload_desc))

    note("CPU oracle baseline" if not args.no_cpu_baseline else "done timing")
    cpu, parity = (None, None) if args.no_cpu_baseline else cpu_baseline(
        cfg, args.cpu_seconds, {"absorb": out_a, "gqa": out_g})
    nxt = next_rows(gqla, rf, cfg, sh, w, gc, dev, args.warmup, K) if flagship else None

    rec = {
        "metric": METRIC,
        "value": round(q_tokens / (ms_per_step * 1e-3), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "settle": settle,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": workload_desc,
                   "batch": B, "ctx": int(cfg.ctx[0]) if cfg.ctx[0] == cfg.ctx[1] else [int(c) for c in cfg.ctx],
                   "h_q": cfg.h_q, "g": cfg.g, "s_q": cfg.s_q, "paths": ["absorb", "gqa"]},
        "paths": paths,
        "roofline": roof,
        "cpu_baseline": cpu,
        "expand_ms": round(expand_ms, 3),
        "next": nxt,
        "parity": parity,
        "input_gen_s": round(t_gen, 1),
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
