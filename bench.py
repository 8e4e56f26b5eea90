#!/usr/bin/env python3
"""Benchmark of the fused DeepSeek-V4 attention prologue on one MI355X.

One step = one call of qnorm_rope_kv_quant_insert over the prefill workload
(32768 tokens x 64 Q heads x 512, one latent KV head per token, 1024 pages of
64 slots; 4,356,540,416 algorithmic bytes).  Inputs are seeded synthetic data
generated on the GPU and resident in HBM before timing starts.

Prints ONE JSON line:
  value        whole-job HBM throughput in GB/s (algorithmic bytes / time)
  pct_of_d2d   value as a fraction of the measured 512 MiB device-to-device
               copy ceiling (read + write bytes counted): the faster of
               hipMemcpyAsync and the library's hand-written 16 B/lane copy
               of the same 512 MiB, both reported with their own ratios;
               beside them its in-place 16 B/lane read-modify-write over 2 GiB
  roofline     dominant kernel: algorithmic bytes per launch / mean launch
               duration (one pair of HIP events on the launch stream around
               the timed launches) against 8 TB/s
  cpu_baseline the CPU oracle timed on a bounded token slice of the same
               workload, single-threaded (cpu_baseline_all_cores: the same
               oracle over disjoint token slices on every core of the share)
  extra        the other workloads (131072 x 64, 32768 x 128, decode and tiny
               latencies, the packed Q/K norm+RoPE at 8192 tokens, the cache
               read side over all 131072 slots of the 131072 x 64 cache, and
               the same prologue as five separate launches, the unfused
               baseline, with the fusion speedup; the packed op at 1024, 4096
               and 8192 tokens against its four separate launches; and the
               pages' grid of 1-131072 tokens at 64 and 128 heads, "sweep").  Each of these launches is
               timed alone after a 1 GiB cache-flushing read (median and
               minimum), so no working set starts in the 256 MB Infinity
               Cache and no dirty line is left to write back;
               prefill_flushed is the headline kernel timed that way.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--quick]
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("achieved HBM GB/s & % of measured D2D-copy peak at tokens×heads "
          "32768×64")
HBM_PEAK_GBPS = 8000.0
PROFILE_COUNTERS = os.path.join(ROOT, "profiles",
                                "dsv4_prologue_prefill_32768x64_counters.json")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


KERNEL_SOURCES = ("dsv4_prologue.hip", "kv_quant.hpp", "wave_ops.hpp")


def kernel_source_hash() -> str:
    """Hash of the code (comments and whitespace removed) of the sources the
    fused prologue kernel is compiled from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp8_kv_cache_slot_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(name.encode() + b"\0" + text.encode())
    return h.hexdigest()[:16]


def measured_traffic(tiling):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources at the tiling in force; else None."""
    try:
        with open(PROFILE_COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None
    if list(c.get("tiling", [])) != list(tiling):
        return None
    return c.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true",
                    help="headline workload only (no extras, no CPU baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the fused prologue is per-token "
              f"independent and has no cross-GPU step, so --gpus {args.gpus} is "
              f"not a configuration of this benchmark", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        sys.exit("--steps must be >= 1")

    import torch

    import fp8_kv_cache_slot_amd as K
    from fp8_kv_cache_slot_amd import accounting as A
    from fp8_kv_cache_slot_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')}")

    # ---- ceiling: 512 MiB device-to-device copy -----------------------------
    n = 512 * 2 ** 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    def back_to_back(fn, iters=20, warmup=3):
        """Mean seconds per call of `iters` back-to-back calls, from one pair
        of events on the launch stream around all of them (an event pair
        around every call adds its own few microseconds to each)."""
        for _ in range(warmup):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(iters):
            fn()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) / 1e3 / iters

    # the same 512 MiB through the library's hand-written 16 B/lane copy, and
    # an in-place 16 B/lane read-modify-write over 2 GiB (the size and access
    # pattern of the prefill Q heads, without the arithmetic)
    d2d_gbps = 2 * n / back_to_back(lambda: dst.copy_(src)) / 1e9
    log(f"hipMemcpyAsync D2D copy {d2d_gbps:.1f} GB/s")
    copy_gbps = 2 * n / back_to_back(lambda: K.stream_copy(dst, src)) / 1e9
    del src, dst
    rbuf = torch.zeros(2 ** 31, dtype=torch.uint8, device=dev)
    rmw_gbps = 2 * rbuf.numel() / back_to_back(lambda: K.stream_rmw(rbuf, 0)) / 1e9
    del rbuf
    log(f"16 B/lane copy kernel {copy_gbps:.1f} GB/s, in-place RMW {rmw_gbps:.1f} GB/s")
    # The D2D-copy ceiling of the metric: the faster of the two measured
    # 512 MiB device-to-device copies (hipMemcpyAsync is the slower one on
    # MI355X, so a ratio against it alone would overstate the kernel).
    ceiling_gbps = max(d2d_gbps, copy_gbps)
    ceiling_src = ("fp8kv_stream_copy (16 B/lane copy kernel)" if copy_gbps > d2d_gbps
                   else "hipMemcpyAsync")

    # 1 GiB read between timed launches: more than the 256 MB Infinity Cache
    # plus the L2s, so every timed launch starts from cold caches.  A read,
    # not a write, leaves the caches clean: after a 1 GiB write the timed
    # launch would also pay for writing back up to 256 MB of the flush's own
    # dirty lines (measured: the 212 MB read side took 59 us after a write
    # flush, 47 us after a read flush).
    flush_buf = torch.ones(2 ** 28, dtype=torch.float32, device=dev)

    def time_flushed(fn, iters=20, warmup=3):
        """Per-launch seconds of `iters` launches, each preceded (outside its
        events) by a 1 GiB cache-flushing read."""
        for _ in range(warmup):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        for a, b in ev:
            flush_buf.sum()
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) / 1e3 for a, b in ev]

    ref_times = {}

    def stream_ref(nbytes, kind):
        """Median seconds of the library's 16 B/lane reference kernel moving
        `nbytes` bytes (read + write), each launch after the same flushing
        read: the in-place RMW over nbytes/2 ("rmw", the access pattern of
        the in-place operators) or a copy of nbytes/2 ("copy")."""
        half = max(16, nbytes // 2 // 16 * 16)
        if (kind, half) not in ref_times:
            a = torch.zeros(half, dtype=torch.uint8, device=dev)
            if kind == "rmw":
                per = time_flushed(lambda: K.stream_rmw(a, 0))
            else:
                b = torch.empty_like(a)
                per = time_flushed(lambda: K.stream_copy(b, a))
                del b
            del a
            torch.cuda.empty_cache()
            ref_times[(kind, half)] = (statistics.median(per), 2 * half)
        return ref_times[(kind, half)]

    def annotate(entry, nb, m, kind):
        """Roofline fields of one workload timed with cold caches: the
        fraction of the 8 TB/s HBM peak, and the same-size reference kernel
        (time ratio: 1.0 = as fast as plain streaming of the same bytes)."""
        r, rb = stream_ref(nb, kind)
        entry["frac_of_hbm_peak"] = round(nb / m / 1e9 / HBM_PEAK_GBPS, 4)
        entry["stream_ref"] = {
            "kernel": "fp8kv_stream_rmw" if kind == "rmw" else "fp8kv_stream_copy",
            "bytes": rb, "median_us": round(r * 1e6, 2),
            "gbps": round(rb / r / 1e9, 1), "frac": round(r / m, 4)}

    cpu_on = not (args.quick or args.no_cpu_baseline)

    def oracle_beside(run, total_units, budget=1.5):
        """CPU-baseline leg for one workload: the oracle, single-threaded, on
        the first n units of the workload, n sized to about `budget` seconds.
        run(n) prepares host copies of the inputs (untimed), times the oracle
        call alone and returns (seconds, algorithmic bytes of the n units)."""
        n = min(total_units, 4)
        dt, _ = run(n)
        n = int(min(total_units, max(n, n * budget / max(dt, 1e-4))))
        dt, nb = run(n)
        return {"gbps": round(nb / dt / 1e9, 4), "units": n,
                "of_units": total_units, "seconds": round(dt, 3), "cores": 1,
                "kind": "oracle"}

    def dsv4_oracle_run(xx, wl, scalar_scale=None):
        """run(n) for oracle_beside: the prologue oracle (blockwise, or the
        scalar-scale convention) on the first n tokens of workload xx."""
        import numpy as np

        import oracle as O
        qw, kw = I.bits(xx["q_weight"]), I.bits(xx["kv_weight"])
        cs = I.bits(xx["cos_sin_cache"])

        def run(n):
            qh, kvh = I.bits(xx["q"][:n]).copy(), I.bits(xx["kv"][:n]).copy()
            ph = I.bits(xx["positions"][:n]).copy()
            sh = I.bits(xx["slot_mapping"][:n]).copy()
            c = np.full((wl.num_pages, 64, 576), I.CACHE_CANARY, np.uint8)
            s = np.full((wl.num_pages, 64, 8), I.SCALE_CANARY, np.uint8)
            written = int(((sh >= 0) & (sh < wl.num_pages * 64)).sum())
            t0 = time.perf_counter()
            if scalar_scale is None:
                O.qnorm_rope_kv_quant_insert(qh, kvh, qw, kw, cs, ph, sh, c, s,
                                             wl.eps)
                nb = A.dsv4_bytes(n, wl.num_heads, written)
            else:
                O.qnorm_rope_kv_quant_insert_scalar(qh, kvh, qw, kw, cs, ph, sh,
                                                    c, scalar_scale, wl.eps)
                nb = A.dsv4_scalar_bytes(n, wl.num_heads, written)
            return time.perf_counter() - t0, nb
        return run

    def unfused_oracle_run(xx, wl):
        """run(n) for oracle_beside: the oracle's separate stages composed as
        the unfused launches are (RMSNorm of q and of kv, RoPE of both,
        quantise+insert), on the first n tokens; bytes are the operator's."""
        import numpy as np

        import oracle as O
        qw, kw = I.bits(xx["q_weight"]), I.bits(xx["kv_weight"])
        cs = I.bits(xx["cos_sin_cache"])

        def run(n):
            qh, kvh = I.bits(xx["q"][:n]).copy(), I.bits(xx["kv"][:n]).copy()
            ph = I.bits(xx["positions"][:n]).copy()
            sh = I.bits(xx["slot_mapping"][:n]).copy()
            c = np.full((wl.num_pages, 64, 576), I.CACHE_CANARY, np.uint8)
            s = np.full((wl.num_pages, 64, 8), I.SCALE_CANARY, np.uint8)
            written = int(((sh >= 0) & (sh < wl.num_pages * 64)).sum())
            t0 = time.perf_counter()
            qn = O.rms_norm_rows(qh, qw, wl.eps)
            kn = O.rms_norm_rows(kvh, kw, wl.eps)
            O.rope_rows(qn, cs, ph)
            O.rope_rows(kn.reshape(n, 1, 512), cs, ph)
            O.kv_quant_insert(kn, sh, c, s)
            return time.perf_counter() - t0, A.dsv4_bytes(n, wl.num_heads, written)
        return run

    def call(x, q, cache, scale):
        K.qnorm_rope_kv_quant_insert(q, x["kv"], x["q_weight"], x["kv_weight"],
                                     x["cos_sin_cache"], x["positions"],
                                     x["slot_mapping"], cache, scale, x["eps"])

    def workload_bytes(w, x):
        sm = x["slot_mapping"]
        written = int(((sm >= 0) & (sm < w.num_pages * 64)).sum().item())
        return A.dsv4_bytes(w.num_tokens, w.num_heads, written)

    def time_launches(fn, steps, warmup):
        """Run warmup untimed launches, then `steps` back-to-back launches
        bracketed by a synchronize on both sides and by one pair of events on
        the launch stream.  Returns (total wall seconds, mean seconds per
        launch from the events).  An event pair around every launch would
        add about 7 us to each 680 us step and 2-3 us to each launch's own
        interval, so the events bracket the whole timed region instead."""
        for _ in range(warmup):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        total = time.perf_counter() - t0
        return total, a.elapsed_time(b) / 1e3 / steps

    # ---- headline: prefill 32768 x 64 ---------------------------------------
    w = I.DSV4_WORKLOADS["prefill"]
    x = I.make_dsv4(w, dev)
    q, cache, scale = x["q"].clone(), x["kv_cache"].clone(), x["kv_scale"].clone()
    nbytes = workload_bytes(w, x)
    total, mean_launch = time_launches(lambda: call(x, q, cache, scale), args.steps,
                                       args.warmup)
    value = nbytes * args.steps / total / 1e9
    achieved = nbytes / mean_launch / 1e9
    log(f"prefill: {value:.1f} GB/s whole-job, kernel {achieved:.1f} GB/s "
        f"({mean_launch * 1e6:.1f} us/launch), {value / ceiling_gbps:.3f} of the "
        f"D2D-copy ceiling")
    traffic = measured_traffic(K.get_tiling())

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "fused DeepSeek-V4 prologue, prefill: 32768 tokens x 64 "
                        "Q heads x 512 (bf16 in/out) + 1 latent KV head -> FP8 "
                        "E4M3 + 7 UE8M0 exponents into 1024 pages x 64 slots",
            "tokens": w.num_tokens, "heads": w.num_heads, "head_dim": 512,
            "rope_dim": 64, "page_size": 64, "num_pages": w.num_pages,
            "algorithmic_bytes": nbytes, "io_dtype": "bf16 -> bf16 q, fp8 e4m3 kv",
            "tiling": list(K.get_tiling()),
            "dispatch_threshold_programs": K.get_dispatch_threshold(),
        },
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "hip": torch.version.hip, "torch": torch.__version__,
                   "cus": props.multi_processor_count},
        "pct_of_d2d": round(value / ceiling_gbps, 4),
        "d2d_ceiling_gbps": round(ceiling_gbps, 1),
        "d2d_ceiling": ceiling_src,
        "d2d_copy_gbps": round(d2d_gbps, 1),
        "pct_of_memcpy_d2d": round(value / d2d_gbps, 4),
        "copy_kernel_gbps": round(copy_gbps, 1),
        "pct_of_copy_kernel": round(value / copy_gbps, 4),
        "rmw_kernel_gbps": round(rmw_gbps, 1),
        "pct_of_rmw_kernel": round(value / rmw_gbps, 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": "dsv4_prologue_kernel<{}, {}, false>".format(*K.get_tiling()),
            "mean_launch_us": round(mean_launch * 1e6, 2),
            "timing": "one pair of HIP events on the launch stream around the "
                      "timed back-to-back launches; mean = their interval / steps",
        },
    }
    # ---- the same call as five separate launches (the unfused baseline) ----
    kv_work = torch.empty((w.num_tokens, 512), dtype=torch.bfloat16, device=dev)

    def unfused():
        K.unfused_prologue(q, x["kv"], x["q_weight"], x["kv_weight"],
                           x["cos_sin_cache"], x["positions"], x["slot_mapping"],
                           cache, scale, x["eps"], kv_work=kv_work)
    fper = time_flushed(lambda: call(x, q, cache, scale), args.steps, args.warmup)
    prefill_flushed = {"median_us": round(statistics.median(fper) * 1e6, 1),
                       "min_us": round(min(fper) * 1e6, 1),
                       "gbps": round(nbytes / statistics.median(fper) / 1e9, 1)}
    annotate(prefill_flushed, nbytes, statistics.median(fper), "rmw")
    log(f"prefill, caches flushed: {prefill_flushed}")
    uper = time_flushed(unfused)
    unfused_prefill = {"median_us": round(statistics.median(uper) * 1e6, 1),
                       "min_us": round(min(uper) * 1e6, 1),
                       "fused_median_us": round(statistics.median(fper) * 1e6, 1),
                       "fusion_speedup": round(statistics.median(uper) /
                                               statistics.median(fper), 3)}
    if cpu_on:
        unfused_prefill["oracle"] = oracle_beside(unfused_oracle_run(x, w),
                                                  w.num_tokens)
    log(f"unfused prefill: {unfused_prefill}")

    # ---- the scalar-scale cache convention on the same workload ----------
    sscale = torch.tensor([0.0173], dtype=torch.float32, device=dev)
    sper = time_flushed(lambda: K.qnorm_rope_kv_quant_insert_scalar_scale(
        q, x["kv"], x["q_weight"], x["kv_weight"], x["cos_sin_cache"],
        x["positions"], x["slot_mapping"], cache, sscale, x["eps"]))
    sm_all = x["slot_mapping"]
    written = int(((sm_all >= 0) & (sm_all < w.num_pages * 64)).sum().item())
    sb = A.dsv4_scalar_bytes(w.num_tokens, w.num_heads, written)
    scalar_prefill = {"median_us": round(statistics.median(sper) * 1e6, 1),
                      "min_us": round(min(sper) * 1e6, 1),
                      "gbps": round(sb / statistics.median(sper) / 1e9, 1)}
    annotate(scalar_prefill, sb, statistics.median(sper), "rmw")
    if cpu_on:
        scalar_prefill["oracle"] = oracle_beside(
            dsv4_oracle_run(x, w, float(sscale.item())), w.num_tokens)
    log(f"scalar-scale prefill: {scalar_prefill}")
    del q, cache, scale, kv_work

    # ---- CPU baseline: the oracle on a bounded slice of the same workload --
    if not (args.quick or args.no_cpu_baseline):
        import numpy as np

        import oracle as O

        def oracle_on(tokens, threads=1):
            """Seconds for the oracle over the first `tokens` prefill tokens,
            split into `threads` disjoint token slices run concurrently (the
            oracle's C entry releases the interpreter lock; the slot map is
            injective, so the slices write disjoint cache rows)."""
            qw, kw = I.bits(x["q_weight"]), I.bits(x["kv_weight"])
            cs = I.bits(x["cos_sin_cache"])
            c = np.full((w.num_pages, 64, 576), I.CACHE_CANARY, np.uint8)
            s = np.full((w.num_pages, 64, 8), I.SCALE_CANARY, np.uint8)
            cuts = [tokens * i // threads for i in range(threads + 1)]
            parts = []
            for a, b in zip(cuts[:-1], cuts[1:]):
                sl = slice(a, b)
                parts.append((I.bits(x["q"][sl]).copy(), I.bits(x["kv"][sl]).copy(),
                              I.bits(x["positions"][sl]).copy(),
                              I.bits(x["slot_mapping"][sl]).copy()))

            def run(p):
                O.qnorm_rope_kv_quant_insert(p[0], p[1], qw, kw, cs, p[2], p[3],
                                             c, s, w.eps)
            t0 = time.perf_counter()
            if threads == 1:
                run(parts[0])
            else:
                with cf.ThreadPoolExecutor(threads) as ex:
                    list(ex.map(run, parts))
            return time.perf_counter() - t0

        probe = 256
        dt = oracle_on(probe)
        tokens = int(min(w.num_tokens, max(probe, probe * args.cpu_seconds / dt)))
        tokens = max(64, tokens // 64 * 64)
        dt = oracle_on(tokens)
        sbytes = A.dsv4_bytes(tokens, w.num_heads, tokens)
        result["cpu_baseline"] = {
            "value": round(sbytes / dt / 1e9, 4),
            "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"first {tokens} of the 32768 prefill tokens (all 64 heads "
                      f"+ KV), {dt:.1f} s single-threaded double-precision C++",
            "seconds": round(dt, 2),
            "host_cpus": os.cpu_count(),
            "cpu_model": cpu_model(),
        }
        log(f"cpu oracle: {tokens} tokens in {dt:.1f} s")
        # every core of this process's CPU share, over disjoint token slices
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
        mt = int(min(w.num_tokens, tokens * threads)) // 64 * 64
        mdt = oracle_on(mt, threads)
        mbytes = A.dsv4_bytes(mt, w.num_heads, mt)
        result["cpu_baseline_all_cores"] = {
            "value": round(mbytes / mdt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {mt} of the 32768 prefill tokens in {threads} "
                      f"disjoint slices, one thread each, {mdt:.1f} s wall",
            "seconds": round(mdt, 2)}
        log(f"cpu oracle, {threads} threads: {mt} tokens in {mdt:.1f} s")

    del x
    torch.cuda.empty_cache()

    # ---- the other workloads -------------------------------------------------
    if not args.quick:
        extra = {}
        for name in ("long64", "wide128"):
            wl = I.DSV4_WORKLOADS[name]
            xx = I.make_dsv4(wl, dev)
            qq, cc, ss = xx["q"].clone(), xx["kv_cache"].clone(), xx["kv_scale"].clone()
            nb = workload_bytes(wl, xx)
            per = time_flushed(lambda: call(xx, qq, cc, ss))
            m = statistics.median(per)
            extra[name] = {"tokens": wl.num_tokens, "heads": wl.num_heads,
                           "bytes": nb, "median_us": round(m * 1e6, 1),
                           "min_us": round(min(per) * 1e6, 1),
                           "gbps": round(nb / m / 1e9, 1),
                           "pct_of_d2d": round(nb / m / 1e9 / ceiling_gbps, 4)}
            annotate(extra[name], nb, m, "rmw")
            if cpu_on:
                extra[name]["oracle"] = oracle_beside(dsv4_oracle_run(xx, wl),
                                                      wl.num_tokens)
            log(f"{name}: {extra[name]}")
            if name == "long64":
                # read side: every slot of the cache just written, in a
                # seeded random order
                g = torch.Generator(device=dev)
                g.manual_seed(7)
                slots = torch.randperm(wl.num_pages * 64, generator=g, device=dev)
                out = torch.empty((slots.shape[0], 512), dtype=torch.bfloat16,
                                  device=dev)
                per = time_flushed(
                    lambda: K.kv_cache_gather_dequant(cc, ss, slots, out))
                m = statistics.median(per)
                nb = A.dequant_bytes(slots.shape[0], slots.shape[0])
                extra["dequant_long64"] = {
                    "rows": int(slots.shape[0]), "bytes": nb,
                    "median_us": round(m * 1e6, 1), "min_us": round(min(per) * 1e6, 1),
                    "gbps": round(nb / m / 1e9, 1)}
                annotate(extra["dequant_long64"], nb, m, "copy")
                if cpu_on:
                    import oracle as O
                    ch, sch = I.bits(cc), I.bits(ss)

                    def dq_run(n):
                        sl = I.bits(slots[:n]).copy()
                        t0 = time.perf_counter()
                        O.kv_cache_gather_dequant(ch, sch, sl)
                        return time.perf_counter() - t0, A.dequant_bytes(n, n)
                    extra["dequant_long64"]["oracle"] = oracle_beside(
                        dq_run, int(slots.shape[0]))
                log(f"dequant_long64: {extra['dequant_long64']}")
                # the scalar-scale read side over the same cache and slots
                rscale = torch.tensor([0.0173], dtype=torch.float32, device=dev)
                per = time_flushed(lambda: K.kv_cache_gather_dequant_scalar_scale(
                    cc, rscale, slots, out))
                m = statistics.median(per)
                nb = A.dequant_scalar_bytes(slots.shape[0], slots.shape[0])
                extra["dequant_scalar_long64"] = {
                    "rows": int(slots.shape[0]), "bytes": nb,
                    "median_us": round(m * 1e6, 1), "min_us": round(min(per) * 1e6, 1),
                    "gbps": round(nb / m / 1e9, 1)}
                annotate(extra["dequant_scalar_long64"], nb, m, "copy")
                if cpu_on:
                    def dqs_run(n):
                        sl = I.bits(slots[:n]).copy()
                        t0 = time.perf_counter()
                        O.kv_cache_gather_dequant_scalar(ch, 0.0173, sl)
                        return time.perf_counter() - t0, A.dequant_scalar_bytes(n, n)
                    extra["dequant_scalar_long64"]["oracle"] = oracle_beside(
                        dqs_run, int(slots.shape[0]))
                log(f"dequant_scalar_long64: {extra['dequant_scalar_long64']}")
                # the same cache read through block tables: 32 sequences of
                # 4096 tokens over all 2048 pages, pages in a seeded order
                S = 32
                pages = wl.num_pages
                table = torch.randperm(pages, generator=g, device=dev).to(
                    torch.int32).view(S, pages // S).contiguous()
                L = pages // S * 64
                lens = torch.full((S,), L, dtype=torch.int32, device=dev)
                offs = torch.arange(S, dtype=torch.int64, device=dev) * L
                per = time_flushed(lambda: K.kv_cache_gather_dequant_paged(
                    cc, ss, table, lens, offs, out))
                m = statistics.median(per)
                nb = A.dequant_paged_bytes(S * L, S * L, pages, S)
                extra["dequant_paged_long64"] = {
                    "rows": S * L, "sequences": S, "bytes": nb,
                    "median_us": round(m * 1e6, 1), "min_us": round(min(per) * 1e6, 1),
                    "gbps": round(nb / m / 1e9, 1)}
                annotate(extra["dequant_paged_long64"], nb, m, "copy")
                if cpu_on:
                    import numpy as np
                    th, lh, oh = I.bits(table), I.bits(lens), I.bits(offs)

                    def dqp_run(n):
                        o = np.zeros((n * L, 512), np.uint16)
                        t0 = time.perf_counter()
                        O.kv_cache_gather_dequant_paged(ch, sch, th[:n], lh[:n],
                                                        oh[:n], o)
                        return (time.perf_counter() - t0,
                                A.dequant_paged_bytes(n * L, n * L,
                                                      n * (pages // S), n))
                    extra["dequant_paged_long64"]["oracle"] = oracle_beside(dqp_run, S)
                log(f"dequant_paged_long64: {extra['dequant_paged_long64']}")
                # the scalar-scale convention through the same block tables
                per = time_flushed(lambda: K.kv_cache_gather_dequant_paged_scalar_scale(
                    cc, rscale, table, lens, offs, out))
                m = statistics.median(per)
                nb = A.dequant_paged_bytes(S * L, S * L, pages, S) - 7 * S * L + 4
                extra["dequant_paged_scalar_long64"] = {
                    "rows": S * L, "sequences": S, "bytes": nb,
                    "median_us": round(m * 1e6, 1), "min_us": round(min(per) * 1e6, 1),
                    "gbps": round(nb / m / 1e9, 1)}
                annotate(extra["dequant_paged_scalar_long64"], nb, m, "copy")
                if cpu_on:
                    def dqps_run(n):
                        o = np.zeros((n * L, 512), np.uint16)
                        t0 = time.perf_counter()
                        O.kv_cache_gather_dequant_paged_scalar(ch, 0.0173, th[:n],
                                                               lh[:n], oh[:n], o)
                        return (time.perf_counter() - t0,
                                A.dequant_paged_bytes(n * L, n * L, n * (pages // S), n)
                                - 7 * n * L + 4)
                    extra["dequant_paged_scalar_long64"]["oracle"] = oracle_beside(
                        dqps_run, S)
                log(f"dequant_paged_scalar_long64: {extra['dequant_paged_scalar_long64']}")
                del slots, out, table, lens, offs
            del xx, qq, cc, ss
            torch.cuda.empty_cache()
        extra["prefill_flushed"] = prefill_flushed
        extra["unfused_prefill"] = unfused_prefill
        extra["scalar_scale_prefill"] = scalar_prefill
        for name in ("tiny", "decode"):
            wl = I.DSV4_WORKLOADS[name]
            xx = I.make_dsv4(wl, dev)
            qq, cc, ss = xx["q"].clone(), xx["kv_cache"].clone(), xx["kv_scale"].clone()
            nb = workload_bytes(wl, xx)
            per = time_flushed(lambda: call(xx, qq, cc, ss), 50, 10)
            m = statistics.median(per)
            kw = torch.empty((wl.num_tokens, 512), dtype=torch.bfloat16, device=dev)
            uper = time_flushed(lambda: K.unfused_prologue(
                qq, xx["kv"], xx["q_weight"], xx["kv_weight"], xx["cos_sin_cache"],
                xx["positions"], xx["slot_mapping"], cc, ss, xx["eps"], kv_work=kw),
                50, 10)
            um = statistics.median(uper)
            extra[name] = {"tokens": wl.num_tokens, "heads": wl.num_heads,
                           "bytes": nb, "median_us": round(m * 1e6, 2),
                           "min_us": round(min(per) * 1e6, 2),
                           "gbps": round(nb / m / 1e9, 1),
                           "unfused_median_us": round(um * 1e6, 2),
                           "fusion_speedup": round(um / m, 3)}
            annotate(extra[name], nb, m, "rmw")
            if cpu_on:
                extra[name]["oracle"] = oracle_beside(dsv4_oracle_run(xx, wl),
                                                      wl.num_tokens)
            log(f"{name}: {extra[name]}")
        # packed at 1 and 17 tokens: launch-bound, reported as latency
        for name in ("packed_t1", "packed_t17"):
            sw = I.PACKED_WORKLOADS[name]
            sx = I.make_packed(sw, dev)
            sq = sx["qkv"].clone()
            per = time_flushed(lambda: K.qk_norm_rope_packed(
                sq, sw.num_heads_q, sw.num_heads_k, sw.num_heads_v, sw.head_dim,
                sw.eps, sx["q_weight"], sx["k_weight"], sx["cos_sin_cache"], True,
                sx["position_ids"]), 50, 10)
            extra[name] = {"tokens": sw.num_tokens, "heads": "16q/8k/8v x 128",
                           "median_us": round(statistics.median(per) * 1e6, 2),
                           "min_us": round(min(per) * 1e6, 2)}
            log(f"{name}: {extra[name]}")
        # packed at the token counts InfiniOps PR #1019 "Benchmark /
        # Performance Impact" measures, fused against its four separate
        # launches (RMSNorm of the Q and of the K heads into preallocated
        # outputs, then RoPE of each)
        for name in ("packed_t1024", "packed_t4096", "packed_t8192"):
            pw = I.PACKED_WORKLOADS[name]
            px = I.make_packed(pw, dev)
            qkv = px["qkv"].clone()

            def pcall():
                K.qk_norm_rope_packed(qkv, pw.num_heads_q, pw.num_heads_k,
                                      pw.num_heads_v, pw.head_dim, pw.eps,
                                      px["q_weight"], px["k_weight"],
                                      px["cos_sin_cache"], True, px["position_ids"])
            per = time_flushed(pcall, 50, 10)
            m = statistics.median(per)
            nb = A.packed_bytes(pw.num_tokens, pw.num_heads_q, pw.num_heads_k,
                                pw.head_dim)
            q_out = torch.empty((pw.num_tokens, pw.num_heads_q, pw.head_dim),
                                dtype=torch.bfloat16, device=dev)
            k_out = torch.empty((pw.num_tokens, pw.num_heads_k, pw.head_dim),
                                dtype=torch.bfloat16, device=dev)
            uper = time_flushed(lambda: K.unfused_qk_norm_rope_packed(
                px["qkv"], pw.num_heads_q, pw.num_heads_k, pw.num_heads_v,
                pw.head_dim, pw.eps, px["q_weight"], px["k_weight"],
                px["cos_sin_cache"], px["position_ids"], q_out, k_out), 50, 10)
            um = statistics.median(uper)
            extra[name] = {"tokens": pw.num_tokens, "heads": "16q/8k/8v x 128",
                           "bytes": nb, "median_us": round(m * 1e6, 2),
                           "min_us": round(min(per) * 1e6, 2),
                           "gbps": round(nb / m / 1e9, 1),
                           "separate_launches_median_us": round(um * 1e6, 2),
                           "fusion_speedup": round(um / m, 3)}
            annotate(extra[name], nb, m, "rmw")
            if cpu_on and name == "packed_t8192":
                import oracle as O
                pqw, pkw = I.bits(px["q_weight"]), I.bits(px["k_weight"])
                pcs, ppos = I.bits(px["cos_sin_cache"]), I.bits(px["position_ids"])

                def pk_run(n):
                    qh = I.bits(px["qkv"][:n]).copy()
                    t0 = time.perf_counter()
                    O.qk_norm_rope_packed(qh, pw.num_heads_q, pw.num_heads_k,
                                          pw.num_heads_v, pw.head_dim, pw.eps, pqw,
                                          pkw, pcs, ppos[:n].copy())
                    return (time.perf_counter() - t0,
                            A.packed_bytes(n, pw.num_heads_q, pw.num_heads_k,
                                           pw.head_dim))
                extra[name]["oracle"] = oracle_beside(pk_run, pw.num_tokens)
            log(f"{name}: {extra[name]}")
            del px, qkv, q_out, k_out
        # packed at long-prefill token counts, where launches of 65536 waves
        # and more run occupancy-capped (7 two-wave blocks per CU)
        for T, seed in ((32768, 1064), (131072, 1074)):
            lw = I.PackedWorkload(f"packed_t{T}", T, seed=seed)
            lx = I.make_packed(lw, dev)
            per = time_flushed(lambda: K.qk_norm_rope_packed(
                lx["qkv"], lw.num_heads_q, lw.num_heads_k, lw.num_heads_v, lw.head_dim,
                lw.eps, lx["q_weight"], lx["k_weight"], lx["cos_sin_cache"], True,
                lx["position_ids"]), 20, 3)
            m = statistics.median(per)
            nb = A.packed_bytes(T, lw.num_heads_q, lw.num_heads_k, lw.head_dim)
            extra[lw.name] = {"tokens": T, "heads": "16q/8k/8v x 128", "bytes": nb,
                              "median_us": round(m * 1e6, 2),
                              "min_us": round(min(per) * 1e6, 2),
                              "gbps": round(nb / m / 1e9, 1)}
            annotate(extra[lw.name], nb, m, "rmw")
            log(f"{lw.name}: {extra[lw.name]}")
            del lx
        # packed variants the guarded fast path does not cover, at 8192 tokens
        # (one wave per block) and at 2048 (a token's four waves in one block)
        for label, D, R, neox, dt, T in [
                ("packed_ex_d64_inter_f16", 64, 64, False, torch.float16, 8192),
                ("packed_ex_d256_neox_r128_bf16", 256, 128, True, torch.bfloat16, 8192),
                ("packed_ex_d256_neox_r128_bf16_t2048", 256, 128, True, torch.bfloat16, 2048)]:
            g = torch.Generator(device=dev)
            g.manual_seed(D + R)
            hq, hk, hv = 16, 8, 8
            vq = torch.randn((T, (hq + hk + hv) * D), generator=g, device=dev).to(dt)
            vw = (torch.rand(D, generator=g, device=dev) + 0.5).to(dt)
            vcs = I.cos_sin_cache(8192, R, device=dev)
            vpos = torch.randint(0, 8192, (T,), generator=g, device=dev)
            per = time_flushed(lambda: K.qk_norm_rope_packed_ex(
                vq, hq, hk, hv, D, 1e-6, vw, vw, vcs, neox, vpos, rotary_dim=R), 50, 10)
            m = statistics.median(per)
            nb = A.packed_bytes(T, hq, hk, D, R)
            extra[label] = {"tokens": T, "heads": f"{hq}q/{hk}k/{hv}v x {D}",
                            "rotary_dim": R, "bytes": nb,
                            "median_us": round(m * 1e6, 2),
                            "min_us": round(min(per) * 1e6, 2),
                            "gbps": round(nb / m / 1e9, 1)}
            annotate(extra[label], nb, m, "rmw")
            if cpu_on:
                import numpy as np

                import oracle as O

                def u16(v):  # bf16 or fp16 bit patterns
                    return v.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
                vwh, vcsh, vph = u16(vw), I.bits(vcs), I.bits(vpos)

                def pex_run(n):
                    qh = u16(vq[:n]).copy()
                    t0 = time.perf_counter()
                    O.qk_norm_rope_packed_ex(qh, hq, hk, hv, D, R, neox,
                                             dt == torch.float16, 1e-6, vwh, vwh,
                                             vcsh, vph[:n].copy())
                    return time.perf_counter() - t0, A.packed_bytes(n, hq, hk, D, R)
                extra[label]["oracle"] = oracle_beside(pex_run, T)
            log(f"{label}: {extra[label]}")
        # the pages' grid (FlagGems PR #5449 "Performance": 1-17, 1024-2048
        # and 8192-131072 tokens at 64 and 128 heads), default dispatch,
        # caches cold: token prefixes of one 131072-token workload per head
        # count (random positions over a 131072-row table, every slot of a
        # 2048-page cache in a random order)
        sweep = {}
        for heads, seed in ((64, 1113), (128, 1123)):
            sw = I.Dsv4Workload(f"sweep{heads}", 131072, heads, 131072, 2048, False,
                                "uniform", "permutation", 0, seed)
            sx = I.make_dsv4(sw, dev)
            for T in (1, 17, 1024, 2048, 8192, 32768, 131072):
                sl = {k: (v[:T] if k in ("q", "kv", "positions", "slot_mapping")
                          else v) for k, v in sx.items()}
                nb = A.dsv4_bytes(T, heads, T)
                per = time_flushed(lambda: call(sl, sl["q"], sl["kv_cache"],
                                                sl["kv_scale"]), 20, 3)
                m = statistics.median(per)
                e = {"tokens": T, "heads": heads, "bytes": nb,
                     "median_us": round(m * 1e6, 2), "min_us": round(min(per) * 1e6, 2),
                     "gbps": round(nb / m / 1e9, 1)}
                annotate(e, nb, m, "rmw")
                sweep[f"{T}x{heads}"] = e
                log(f"sweep {T}x{heads}: {e['median_us']} us, {e['gbps']} GB/s, "
                    f"ref {e['stream_ref']['frac']}")
            del sx, sl
            torch.cuda.empty_cache()
        extra["sweep"] = sweep
        result["extra"] = extra

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
