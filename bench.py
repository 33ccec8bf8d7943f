#!/usr/bin/env python3
"""ADA paged-decode benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gqa_t32k]

One step is one ska_decode_attention call over the whole batch: one kernel
that prepares the query codes, streams the pages (logits from angle codes,
online softmax, bf16 value accumulation) and merges the splits.  Inputs are
resident in HBM before the timed region; two copies of the page pools are
alternated so that the 256 MB Infinity Cache cannot serve one step's pages to
the next.  Each measured path first runs --settle untimed steps back to back
(the GPU's clock controller needs about 20 ms of this load to settle after an
idle period), then the W warm-up steps, then the K timed steps,
uninstrumented; a further pass, settled the same way, times the decode
kernel itself: one more HIP event after its first step, and the span of the
K-1 calls after it, which run back to back.  The line also reports the K
steps timed right after the encode, before any settling
(cold_start_us_per_step).

dtype: the step computes in binary32 (logits, softmax, accumulation) with the
query direction entering f_b as binary16 and the values and probabilities
entering P.V as bf16 (P split exactly into two bf16 halves).

Prints one JSON line (stdout): effective HBM GB/s on algorithmic bytes (the
compressed bytes the method must read), KV tokens/s, the decode kernel's
roofline figures and the CPU oracle's throughput on a bounded sample.
Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["long_context_decode_ada_amd/csrc/k_decode.h", "long_context_decode_ada_amd/csrc/k_decode.hip",
                  "long_context_decode_ada_amd/csrc/ska_codes.h",
                  "long_context_decode_ada_amd/csrc/ska_internal.h"]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def decode_kernel_bytes(w) -> int:
    """Algorithmic bytes the decode kernel must read in one launch: per
    resident (token, kv head) the record, the radius byte and d bf16 values;
    per resident (page, kv head) the block-table entry and the page header
    (and the 8-byte page offset when pages have variable size)."""
    return w.bytes_per_step() - w.B * w.hq * w.d * 4 * 2


def read_traffic(workload: str):
    """HBM bytes per decode launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source (else None)."""
    path = os.path.join(PROFILES, "k_decode_%s_pmc.md" % workload)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("- ") and " = " in line:
            k, v = line[2:].split(" = ", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha") != kernel_source_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, nseq: int, min_seconds: float):
    """The CPU oracle (plain fp64 C, all host threads) on the first `nseq`
    sequences of the workload: encode untimed, then the decode of those
    sequences (all query heads) repeated until `min_seconds` have passed."""
    import numpy as np
    from long_context_decode_ada_amd import workloads as W
    from oracle import oracle as O
    # the first nseq sequences (their keys are the first rows of w.keys)
    sub = W.Workload(**{**w.__dict__, "B": nseq, "seq_lens": w.seq_lens[:nseq], "block_table": w.block_table[:nseq],
                        "q": w.q[:nseq]})
    ntok = sub.n_tokens
    rng = O.calibrate(w.keys)
    pools = W.host_pools(w, poison=False)
    rows = slice(0, ntok)
    O.encode(pools, w.keys[rows], w.values[rows], w.slot[rows], w.radius_mode, rng)
    pairs = [(s, h) for s in range(nseq) for h in range(w.hq)]
    reps, t0 = 0, time.perf_counter()
    while True:
        O.decode(pools, w.radius_mode, rng, w.q, w.block_table, w.seq_lens, pairs=pairs)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= 100:
            break
    nbytes = reps * (sub.bytes_per_step() - nseq * w.hq * w.d * 8)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": O.max_threads(), "kind": "oracle",
            "kv_tokens_per_s": reps * ntok / dt, "seconds": dt,
            "sample": "%d of %d sequences of %s (%d tokens, all %d query heads), decode only, %d passes" %
                      (nseq, w.B, w.name, ntok, w.hq, reps)}


def context_sweep(args, torch, ska, W):
    """ADA and dense-bf16 decode steps at T = 8K, 32K and 128K with gqa_t32k's
    batch shape (B=8, 32/8 heads, d=128, b=4, shuffled pages).  Keys and
    values are drawn N(0,1) on the GPU (the times do not depend on their
    values); two pool copies alternate as in the main measurement, and each
    path settles (about 45 ms of its steps) before its warm-up and timed
    steps."""
    dev = "cuda"
    res = []
    for T in (8192, 32768, 131072):
        w = W.make("gqa_t32k", T / 32768.0, data=False)
        g = torch.Generator(device=dev)
        g.manual_seed(T)
        slot = torch.from_numpy(w.slot).to(dev)
        caches, kd, rng = [], [], None
        for c in range(2):
            keys = torch.randn((w.n_tokens, w.hkv, w.d), device=dev, generator=g)
            vals = torch.randn((w.n_tokens, w.hkv, w.d), device=dev, generator=g).to(torch.bfloat16).view(torch.int16)
            cache = ska.Cache(ska.DevicePools.for_workload(w, device=dev, poison=False))
            ska.encode_keys(cache, keys, vals, slot, radius_range=rng)
            rng = ska.radius_range(cache)
            k = torch.zeros((w.num_pages, w.hkv, 16, w.d), dtype=torch.bfloat16, device=dev)
            k[slot // 16, :, slot % 16, :] = keys.to(torch.bfloat16)
            caches.append(cache)
            kd.append(k.view(torch.int16))
            del keys, vals
        q = torch.randn((w.B, w.hq, w.d), device=dev, generator=g)
        bt = torch.from_numpy(w.block_table).to(dev)
        sl = torch.from_numpy(w.seq_lens).to(dev)
        out = torch.empty((w.B, w.hq, w.d), dtype=torch.float32, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def timed(fn, steps):
            # settle as the main measurement does: about 45 ms of this path's
            # steps back to back (the count from a short timing), then the
            # warm-up and the timed steps
            for i in range(5):
                fn(i)
            torch.cuda.synchronize()
            e0.record()
            for i in range(5):
                fn(i)
            e1.record()
            torch.cuda.synchronize()
            settle = int(math.ceil(45.0 / max(1e-3, e0.elapsed_time(e1) / 5)))
            for i in range(settle + args.warmup):
                fn(i)
            torch.cuda.synchronize()
            e0.record()
            for i in range(steps):
                fn(i)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / steps

        steps = max(20, args.steps // 2)
        # (each call's arguments checked and marshalled once, before timing)
        ada_calls = [ska.prepared_decode(c, q, bt, sl, out) for c in caches]
        dense_calls = [ska.prepared_decode(c, q, bt, sl, out, k_dense=k) for c, k in zip(caches, kd)]
        ms_ada = timed(lambda i: ada_calls[i % 2](), steps)
        ms_dense = timed(lambda i: dense_calls[i % 2](), steps)
        ada_b = w.bytes_per_step()
        res_t = w.n_tokens * w.hkv
        dense_b = res_t * 4 * w.d + sum((int(n) + 15) // 16 for n in w.seq_lens) * w.hkv * 4 + w.B * w.hq * w.d * 8
        res.append({"T": T, "ada_us": round(ms_ada * 1e3, 2), "ada_GB/s": round(ada_b / (ms_ada * 1e-3) / 1e9, 1),
                    "dense_bf16_us": round(ms_dense * 1e3, 2),
                    "dense_GB/s": round(dense_b / (ms_dense * 1e-3) / 1e9, 1),
                    "ada_speedup": round(ms_dense / ms_ada, 3)})
        log("context T=%d: ADA %.2f us, dense %.2f us (x%.2f)" % (T, ms_ada * 1e3, ms_dense * 1e3, ms_dense / ms_ada))
        for c in caches:
            c.free()
        del caches, kd
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    # After an idle period the GPU's clock controller runs this load fast for
    # about 2 ms, then lowers the clock for about 15 ms before it settles; the
    # untimed settling steps before the W warm-up steps bring each measured
    # path to that steady state (about 45 ms of decode steps).
    ap.add_argument("--settle", type=int, default=0,
                    help="untimed steps run back to back before the warm-up of each measured path "
                         "(0: as many as take --settle-ms)")
    ap.add_argument("--settle-ms", type=float, default=45.0,
                    help="settling time of each measured path when --settle is 0")
    ap.add_argument("--workload", default="gqa_t32k")
    ap.add_argument("--copies", type=int, default=2, help="pool copies alternated across steps")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--cpu-seqs", type=int, default=8, help="sequences in the CPU-oracle sample (0: skip)")
    ap.add_argument("--sweep-context", action="store_true",
                    help="also time ADA and dense bf16 at T = 8K, 32K, 128K with gqa_t32k's batch shape")
    ap.add_argument("--no-baselines", action="store_true",
                    help="skip the dense-bf16 and decompress-then-dot timings on the same pages")
    ap.add_argument("--head-tiers", action="store_true",
                    help="mixed_tiers only: a tier per (page, KV head) instead of per page")
    ap.add_argument("--query-precision", choices=("f16", "f32"), default="f16",
                    help="precision of the query direction inside f_b (the pool's query_precision)")
    ap.add_argument("--no-append", action="store_true",
                    help="skip the timing of the decode step with append (ska_append_decode_attention)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum CPU-oracle timing")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run a plain copy kernel of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this benchmark measures one GPU only (the decode needs no inter-GPU "
              "communication); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from long_context_decode_ada_amd import ska
    from long_context_decode_ada_amd import workloads as W

    t0 = time.time()
    if args.workload == "mixed_tiers_rdr":
        # tiers and evictions planned by the library's RDR controller
        inp = W.rdr_inputs()
        plan = ska.rdr_plan(*(torch.from_numpy(a).to("cuda") for a in (inp.utility, inp.key_norm, inp.protect,
                                                                          inp.num_states, inp.budget)),
                            inp.tiers, inp.eps, inp.bytes_per_tier, inp.sigma)
        plan = {k: v.cpu().numpy() for k, v in plan.items()}
        w = W.planned_workload(inp, plan["tier"], plan["page"], plan["slot"],
                               [plan["page_tier"][s, : int(plan["npages"][s])] for s in range(inp.base.B)],
                               plan["npages"])
        del inp
    else:
        w = W.make(args.workload, head_tiers=args.head_tiers)
    log("workload %s: B=%d hq=%d hkv=%d d=%d tokens=%d pages=%d (%.1fs)" %
        (w.name, w.B, w.hq, w.hkv, w.d, w.n_tokens, w.num_pages, time.time() - t0))
    dev = "cuda"
    keys = torch.from_numpy(w.keys).to(dev)
    vals = torch.from_numpy(w.values.view(np.int16)).to(dev)
    slot = torch.from_numpy(w.slot).to(dev)
    caches, rng = [], None
    qprec = ska.QDIR_F32 if args.query_precision == "f32" else ska.QDIR_F16
    for c in range(args.copies):
        pools = ska.DevicePools.for_workload(w, device=dev, poison=False, max_splits=args.splits,
                                             query_precision=qprec)
        cache = ska.Cache(pools)
        ska.encode_keys(cache, keys, vals, slot, radius_range=rng)
        rng = ska.radius_range(cache)
        caches.append(cache)
    del vals
    # dense bf16 key pools for the baselines (token-major [num_pages][hkv][16][d]), one per pool copy
    kdense = []
    if not args.no_baselines:
        for c in range(args.copies):
            kd = torch.zeros((w.num_pages, w.hkv, 16, w.d), dtype=torch.bfloat16, device=dev)
            kd[slot // 16, :, slot % 16, :] = keys.to(torch.bfloat16)
            kdense.append(kd.view(torch.int16))
    del keys, slot
    torch.cuda.synchronize()
    log("encoded %d pool copies (%.1fs)" % (args.copies, time.time() - t0))
    q = torch.from_numpy(w.q).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    out = torch.empty((w.B, w.hq, w.d), dtype=torch.float32, device=dev)
    nc = len(caches)

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)

    def settle_for(fn):
        """The settling steps of a path: --settle, or as many as take
        --settle-ms at the path's own step time (timed on a few steps)."""
        if args.settle > 0:
            return args.settle
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(5):
            fn(i)
        ev1.record()
        torch.cuda.synchronize()
        return int(math.ceil(args.settle_ms / max(1e-3, ev0.elapsed_time(ev1) / 5)))

    def measure(fn, steps, settle):
        """`settle` untimed steps back to back, then the W warm-up steps,
        then EXACTLY `steps` timed steps between two HIP events, bracketed by
        device synchronisations; ms per step."""
        for i in range(settle):
            fn(i)
        for i in range(args.warmup):
            fn(settle + i)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(steps):
            fn(i)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps

    evm = torch.cuda.Event(enable_timing=True)

    def kernel_span(fn, steps, settle):
        """As measure(), with one more event after the first timed step:
        ms per step over the steps after it."""
        for i in range(settle):
            fn(i)
        for i in range(args.warmup):
            fn(settle + i)
        torch.cuda.synchronize()
        ev0.record()
        fn(0)
        evm.record()
        for i in range(1, steps):
            fn(i)
        ev1.record()
        torch.cuda.synchronize()
        if steps < 2:
            return ev0.elapsed_time(ev1)
        return evm.elapsed_time(ev1) / (steps - 1)

    # one decode step per call; its arguments are checked and marshalled once,
    # here, so that a timed step enqueues only the library call
    ada_calls = [ska.prepared_decode(c, q, bt, sl, out, num_splits=args.splits) for c in caches]

    def run_ada(i):
        ada_calls[i % nc]()

    # Cold start: W warm-up steps and K steps straight after the encode (the
    # GPU idle before).  Reported, not the metric: after an idle period the
    # clock controller lets the first ~2 ms of this load run fast, then lowers
    # the clock for ~15 ms and settles (per-launch kernel trace; a plain copy
    # kernel shows no such transient, see the design notes).
    ms_cold = measure(run_ada, args.steps, 0)
    # The metric: `settle` untimed steps (about 45 ms of this load) bring the
    # GPU to its steady state, then the W warm-up and the K timed steps.
    settle = settle_for(run_ada)
    ms_per_step = measure(run_ada, args.steps, settle)
    # The decode kernel's own average duration, after the same settling and
    # warm-up: K steps between HIP events on the launch stream, with one
    # more event after the first step.  The K-1 calls after that event run
    # back to back (in the kernel trace one kernel starts as the previous
    # ends), so their span divided by K-1 is the kernel's average launch
    # duration without the latency of the first launch after the start
    # event.  (An event pair around every kernel would add each marker's
    # dispatch latency, about 5 us, to every launch.)  With a unit-order
    # kernel in the step (batches of several rounds) the span covers it too.
    k_ms = kernel_span(run_ada, args.steps, settle)
    log("timed %d steps: %.2f us/step (cold start: %.2f); decode kernel %.2f us (back to back, HIP events)"
        % (args.steps, ms_per_step * 1e3, ms_cold * 1e3, k_ms * 1e3))
    if not np.isfinite(out.cpu().numpy()).all():
        log("non-finite output")
        sys.exit(1)

    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log("copy kernel: %d MiB read + %d MiB written, 3 launches" % (args.copy_calib_mib, args.copy_calib_mib))

    step_bytes = w.bytes_per_step()
    ms_per_step = float(ms_per_step)
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    kb = decode_kernel_bytes(w)
    ach = float(kb / (k_ms * 1e-3) / 1e9)
    # (the counter summaries cover the binary16-direction kernel)
    traffic = read_traffic(w.name) if args.query_precision == "f16" else None
    roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic,
            "kernel": "k_decode<d=%d,G=%d>" % (w.d, w.hq // w.hkv), "kernel_us": round(k_ms * 1e3, 2),
            "kernel_us_method": "HIP events: span of K-1 back-to-back calls after the first timed one",
            "alg_bytes_per_launch": int(kb)}

    baselines = None
    if kdense:
        # the same pages read by the two paths the codes are set against: dense
        # bf16 keys, and decompress-then-dot (r~ u(c) written to a dense pool,
        # then the dense decode); values, block table and query as above
        dense_calls = [ska.prepared_decode(c, q, bt, sl, out, num_splits=args.splits, k_dense=k)
                       for c, k in zip(caches, kdense)]

        def run_dense(i):
            dense_calls[i % nc]()

        def run_dtd(i):
            ska.decompress_keys(caches[i % nc], bt, sl, kdense[i % nc])
            dense_calls[i % nc]()

        res_t = w.n_tokens * w.hkv                      # resident (token, KV head) units
        pages_kv = sum((int(n) + 15) // 16 for n in w.seq_lens) * w.hkv
        qo = w.B * w.hq * w.d * 4 * 2
        dense_bytes = res_t * 4 * w.d + pages_kv * 4 + qo
        # the decompress kernel reads the codes, radius bytes, block table and
        # headers (the coded step's bytes without values, query and output)
        code_bytes = step_bytes - qo - res_t * 2 * w.d
        dtd_bytes = code_bytes + res_t * 2 * w.d + dense_bytes
        ms_dense = float(measure(run_dense, args.steps, settle_for(run_dense)))
        ms_dtd = float(measure(run_dtd, args.steps, settle_for(run_dtd)))
        log("baselines: dense bf16 %.2f us/step, decompress-then-dot %.2f us/step" % (ms_dense * 1e3, ms_dtd * 1e3))
        baselines = {
            "dense_bf16": {"us_per_step": round(ms_dense * 1e3, 2), "bytes_per_step": int(dense_bytes),
                           "GB/s": round(dense_bytes / (ms_dense * 1e-3) / 1e9, 1)},
            "decompress_then_dot": {"us_per_step": round(ms_dtd * 1e3, 2), "bytes_per_step": int(dtd_bytes),
                                    "GB/s": round(dtd_bytes / (ms_dtd * 1e-3) / 1e9, 1)},
            "ada_speedup": {"vs_dense_bf16": round(ms_dense / ms_per_step, 3),
                            "vs_decompress_then_dot": round(ms_dtd / ms_per_step, 3)},
        }

    append = None
    if not args.no_append:
        # the decode step with append: each sequence's token at position
        # seq_len - 1 is encoded into its slot (a synthetic new token over the
        # last one resident), then the same decode
        g = torch.Generator(device=dev)
        g.manual_seed(7)
        nk = torch.randn((w.B, w.hkv, w.d), device=dev, generator=g)
        nv = torch.randn((w.B, w.hkv, w.d), device=dev, generator=g).to(torch.bfloat16).view(torch.int16)

        def run_append(i):
            ska.append_decode_attention(caches[i % nc], nk, nv, q, bt, sl, num_splits=args.splits, out=out)

        ms_app = measure(run_append, args.steps, settle_for(run_append))
        log("decode step with append: %.2f us/step" % (ms_app * 1e3))
        append = {"us_per_step": round(ms_app * 1e3, 2), "extra_us_vs_decode": round((ms_app - ms_per_step) * 1e3, 2)}

    sweep = None
    if args.sweep_context:
        del caches, kdense
        torch.cuda.empty_cache()
        sweep = context_sweep(args, torch, ska, W)

    cpu = None
    if args.cpu_seqs > 0:
        log("timing the CPU oracle on %d sequences" % args.cpu_seqs)
        cpu = cpu_baseline(w, min(args.cpu_seqs, w.B), args.cpu_seconds)
        log("oracle: %.3f GB/s (%.1fs, %d threads)" % (cpu["value"], cpu["seconds"], cpu["cores"]))

    tiers = sorted({int(b) for b in np.unique(w.page_bits)})
    line = {
        "metric": "ADA decode effective HBM GB/s (% of peak) and KV tokens/s at T=32k",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32+fp16+bf16" if args.query_precision == "f16" else "fp32+bf16",
        "data": "synthetic",
        "pct_of_peak_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "kv_tokens_per_s": round(w.n_tokens / (ms_per_step * 1e-3), 1),
        "token_kvhead_per_s": round(w.n_tokens * w.hkv / (ms_per_step * 1e-3), 1),
        "alg_bytes_per_step": int(step_bytes),
        "settle_steps": settle,
        "cold_start_us_per_step": round(ms_cold * 1e3, 2),
        "config": {"workload": w.name + (" (tier per page and KV head)" if w.head_tiers else ""),
                   "B": w.B, "hq": w.hq, "hkv": w.hkv, "d": w.d,
                   "T": int(w.seq_lens.max()), "angle_bits": tiers, "radius": "8-bit " +
                   ("log" if w.radius_mode == W.LOG else "uniform"), "page": 16,
                   "values": "bf16", "pool_copies": nc, "splits": args.splits or "auto",
                   "query_direction": "binary16" if args.query_precision == "f16" else "binary32"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "baselines": baselines,
        "append_step": append,
        "context_sweep": sweep,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
