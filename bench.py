#!/usr/bin/env python3
"""Benchmark of the per-GPU Ulysses attention front end on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input of
the 56-head, Ulysses-4 shard (B=1, S_local=9472, H=56, hidden=7168, bshd,
schedule [2, 10, 2]):
  * qkvx_forward: fused QKV projection + RMSNorm(Q, K) + RoPE + head-band store
    into the 4 receive slots (host validation and planning included);
  * ulysses_pack_qkv_head_chunk for every chunk of the schedule, into the 4
    receive slots at rows rank*S_local..;
  * ulysses_merge_output_head_chunk for every chunk, from a seeded attention
    output band [1, 37888, 14, 128] into [1, 9472, 56, 128].
Inputs are resident in HBM before the timed region.  ``value`` is the step's
algorithmic projection FLOPs (2*M*N*K) over the step time; per-kernel times
come from HIP events recorded on the launch stream inside the timed region.

Prints one JSON line.  Only --gpus 1 is supported (one GPU's share of the
exchange; the peers are simulated in local HBM).  --workload runs the same
step on another of the named workloads (for counter profiles of those shapes);
the reported metric is quoted on the 56-head Ulysses-4 shard.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "h56_u4"               # the shard the metric is quoted on
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"fused_qkvx_{workload}_traffic.txt")


def mfma_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"fused_qkvx_{workload}_mfma.txt")


# the fused kernel's code: its source and the internal header with its tile
# order and argument block
FUSED_SOURCES = tuple(os.path.join(ROOT, "head_exchange_amd", "csrc", f)
                      for f in ("qkvx_fused.hip", "qkvx_internal.h"))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--workload", default=WORKLOAD,
                   choices=["h32_u4_fused", "h56_u4", "h56_u2_fused", "h48_u8_stress"],
                   help="workload of the step (default: the 56-head Ulysses-4 shard)")
    p.add_argument("--steps", type=int, default=20)
    # 25 steps (~55 ms) let the clocks settle at this load; after 5 the first
    # timed steps still ran 2-5 % slower
    p.add_argument("--warmup", type=int, default=25)
    p.add_argument("--skip-cpu-baseline", action="store_true",
                   help="do not time the CPU oracle (for profiler runs)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target duration of the CPU oracle sample")
    p.add_argument("--skip-sweep", action="store_true",
                   help="do not time the other workloads and the cold-cache launches")
    p.add_argument("--skip-power", action="store_true",
                   help="do not sample power and clocks with amd-smi (for profiler runs: the "
                        "tool is a script whose launcher replaces itself with its interpreter, "
                        "which a process under the profiler's preload must not do)")
    return p.parse_args()


def source_hash(paths=FUSED_SOURCES) -> str:
    """sha256[:16] of C++/HIP sources with their comments and blank lines taken
    out, so that a counter summary stays attached to the code it measured
    through edits of the comments alone."""
    import re
    h = hashlib.sha256()
    for path in paths:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
        h.update("\n".join(ln for ln in lines if ln.strip()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def profile_label(path: str) -> str:
    """Where a figure read from a committed counter summary comes from."""
    return f"{os.path.relpath(path, ROOT)} @ kernel code {source_hash()}"


def read_traffic(workload: str):
    """HBM bytes per launch of the fused kernel from the committed counter
    summary, or None when it is missing or the kernel changed since."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, x, w, wq, wk, cs, qkv_src, band, target_s: float):
    """The oracle, as it is, on a bounded sample of the same step: the first T
    tokens of the shard through projection + norm + RoPE + rounding + placement,
    and the pack and merge index maps of those T tokens for every chunk."""
    import oracle as O
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    M, N, K = wl.gemm_shape
    S, U, hl = wl.s_local, wl.world, wl.local_heads
    sched = W.schedule_pairs(wl.schedule)

    parts = {}

    def step(T):
        t0 = time.perf_counter()
        xs = x[:, :T]
        vals = O.front_end_values(xs, w, wq, wk, cs, wl.heads, wl.rank)
        O.receive_slots(vals, U, wl.rank)
        t1 = time.perf_counter()
        q, k, v = (a[:, :T] for a in qkv_src)
        for off, cnt in sched:
            dests = [np.empty((wl.batch, T, cnt, 384), np.uint16) for _ in range(U)]
            O.pack_qkv_head_chunk_into(q, k, v, U, off, cnt, dests, 0)
        t2 = time.perf_counter()
        out = np.empty((wl.batch, T, wl.heads, 128), np.uint16)
        srcs = [band[:, u * S:u * S + T] for u in range(U)]
        for off, cnt in sched:
            O.merge_output_head_chunk(srcs, 0, off, U, hl, off, cnt, out)
        t3 = time.perf_counter()
        parts.update(fused=t1 - t0, pack=t2 - t1, merge=t3 - t2)
        return t3 - t0

    step(64)                                     # warm-up (allocations, BLAS threads)
    t_a, t_b = step(64), step(256)
    per_token = max((t_b - t_a) / 192.0, 1e-6)
    fixed = max(t_a - 64 * per_token, 0.0)
    T = int(min(S, max(256, (target_s - fixed) / per_token)))
    T = max(64, (T // 64) * 64)
    dt = step(T)
    flops = 2.0 * wl.batch * T * N * K
    pack_bytes = sum(2.0 * wl.batch * T * U * cnt * 384 * 2 for _, cnt in sched)
    merge_bytes = sum(2.0 * wl.batch * T * U * cnt * 128 * 2 for _, cnt in sched)
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "host_cpus": os.cpu_count(), "usable_cpus": usable, "cpu_model": model,
            "threads_note": "cores = BLAS threads of the float64 projection; the rest of the "
                            "oracle runs on one thread",
            "fused_tflops": flops / parts["fused"] / 1e12,
            "pack_gbps": pack_bytes / parts["pack"] / 1e9,
            "merge_gbps": merge_bytes / parts["merge"] / 1e9,
            "sample": f"first {T} of {S} tokens of the shard: float64 projection, RMSNorm, RoPE, "
                      f"bf16 rounding and receive-slot placement, plus the pack and merge index "
                      f"maps of those tokens for all {len(sched)} chunks; {dt:.1f} s wall",
            "seconds": round(dt, 2), "tokens": T}


SWEEP = ["h32_u4_fused", "h56_u4", "h56_u2_fused", "h48_u8_stress"]
EVICT_BYTES = 1 << 30           # > the 256 MB MALL and the 8 x 4 MB L2s


def read_mfma_counters(workload: str):
    """MFMA busy fraction and shader clock of the fused kernel from the committed
    counter summary, or None when it is missing or the kernel changed since."""
    path = mfma_file(workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    if source_hash() not in text:
        return None
    kv = {}
    for line in text.splitlines():
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip().split()[0]
    try:
        return {"mfma_busy_frac": float(kv["mfma_busy_fraction"]),
                "clock_ghz": float(kv["clock_ghz"])}
    except (KeyError, ValueError):
        return None


def pct(ms):
    """Median and 10th/90th percentiles of per-launch times, in microseconds."""
    a = np.asarray(ms, dtype=np.float64) * 1e3
    return {"p10_us": float(np.percentile(a, 10)), "median_us": float(np.median(a)),
            "p90_us": float(np.percentile(a, 90))}


def evict_caches(torch, evict):
    """Read the 1 GiB buffer ``evict`` (more than the 256 MB MALL and the 8 x 4 MB
    L2s; a float32 sum, which reads it in ~0.27 ms): afterwards the caches hold
    clean lines of it and none of the next kernel's inputs.  (A write fill would
    leave dirty lines whose write-back then falls inside the next timed
    region.)"""
    return evict.view(torch.float32).sum()


WARMUP_S = 0.05                # device time of warm-up launches before a timed series


def warm_up(torch, fn, seconds: float = WARMUP_S) -> None:
    """Run ``fn`` back to back for about ``seconds`` so that the clocks settle
    at the steady state of this load (after an idle gap the first milliseconds
    run at another clock than the rest: a 0.37 ms kernel timed right away
    measured 20 % slower than later in the same process)."""
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    per = max((time.perf_counter() - t0) / 3, 1e-5)
    for _ in range(int(seconds / per)):
        fn()
    torch.cuda.synchronize()


def launch_times(torch, fn, reps: int, stream, lead, evict=None):
    """Per-launch times (ms) from HIP events recorded on the launch stream around
    each launch (for kernels of a millisecond or more: a pair of events costs a
    few microseconds).  With ``evict`` (a 1 GiB device buffer) each launch is
    preceded by a read of that buffer, so its inputs start outside the MALL and
    L2s.  A lead fill of ``lead`` queues ahead of the first launch so that the
    host stays ahead of the device and no enqueue latency falls between a
    launch's events."""
    warm_up(torch, fn)
    lead.fill_(0)
    evs = []
    for i in range(reps):
        if evict is not None:
            evict_caches(torch, evict)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


LEAD_CYCLES = 4_000_000       # a spin of about 2 ms queued ahead of timed launches


def back_to_back_us(torch, fn, stream, reps: int = 20) -> float:
    """Mean time of ``fn`` (one or several launches) run ``reps`` times back to
    back between one pair of events: no per-launch event cost.  A spin kernel
    queued first (it touches no memory) keeps the device busy while the host
    enqueues the launches, so that short kernels are not timed at the rate the
    host issues them (about 12 us per call through the Python binding)."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(LEAD_CYCLES)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def cold_us(torch, fn, stream, evict, reps: int = 10, rounds: int = 5) -> float:
    """Time of ``fn`` (one or several launches) when its inputs come from HBM:
    ``reps`` x (read of the 1 GiB ``evict`` buffer, then ``fn``) back to back
    between one pair of events, minus ``reps`` reads alone, per rep; median over
    ``rounds`` alternating pairs of series.  Launches stay back to back, so
    no pair of events falls around a short kernel (a pair around a near-empty
    kernel measures ~6 us, against ~2 us for the same kernel back to back)."""
    ev = lambda: evict_caches(torch, evict)

    def both():
        ev()
        fn()

    alone, with_fn = [], []
    for _ in range(rounds):
        alone.append(back_to_back_us(torch, ev, stream, reps))
        with_fn.append(back_to_back_us(torch, both, stream, reps))
    return float(np.median(with_fn) - np.median(alone))


def copy_sizes(wl) -> dict:
    """1 GiB, and the read bytes of each distinct merge chunk of the workload."""
    import workloads as W
    sizes = {"1GiB": 1 << 30}
    for _, cnt in W.schedule_pairs(wl.schedule):
        sizes[f"merge_chunk_{cnt}_heads"] = wl.batch * wl.s_local * wl.world * cnt * 256
    return sizes


def copy_ceiling(torch, dev, stream, evict, wl):
    """The practical HBM ceiling: plain contiguous device-to-device copies, back
    to back and from HBM (``cold_us``); bytes read + written.  At 1 GiB: torch's
    copy kernel and the library's 16-byte streaming copy (the exchange_chunks
    kernel with one peer); at the byte counts of the merge chunks: the library
    copy, which shows what a launch of that size reaches from HBM at best."""
    import head_exchange_amd as hx
    out = {}
    for label, size in copy_sizes(wl).items():
        src = torch.empty(size, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        nbytes = 2.0 * size
        cases = {"library_copy": lambda: hx.ulysses_exchange_chunks(
            src.view(1, -1), world=1, rank=0, dst=[dst.view(1, -1)], stream=stream)}
        if label == "1GiB":
            cases["torch_copy"] = lambda: dst.copy_(src)
        res = {"bytes": nbytes}
        for name, fn in cases.items():
            warm = back_to_back_us(torch, fn, stream, 10)
            cold = cold_us(torch, fn, stream, evict)
            res[name] = {"warm_us": warm, "warm_gbps": nbytes / (warm * 1e-6) / 1e9,
                         "warm_frac": nbytes / (warm * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                         "cold_us": cold, "cold_gbps": nbytes / (cold * 1e-6) / 1e9,
                         "cold_frac": nbytes / (cold * 1e-6) / 1e9 / PEAK_HBM_GBPS}
        out[label] = res
        del src, dst
        torch.cuda.empty_cache()
    return out


def device_normal(torch, dev, shape, std: float, seed: int):
    """Seeded N(0, std) bf16 drawn on the device (torch's Philox generator), for
    timing inputs only: same shapes and distributions as the workload recipe."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std).to(
        torch.bfloat16)


def sweep(hx, torch, W, dev, reps: int = 10):
    """Every multi-head workload at its full size: the fused kernel per launch
    (warm, and after a read of a 1 GiB buffer: cold), pack and merge per chunk
    back to back, and the whole schedule of chunks as one group, warm and cold.
    Rates use the algorithmic work: 2*M*N*K for the fused kernel, bytes read +
    written by the band copy for pack and merge."""
    stream = torch.cuda.current_stream()
    evict = torch.empty(EVICT_BYTES, dtype=torch.uint8, device=dev)
    evict.fill_(3)
    out = {}
    for name in SWEEP:
        wl = W.WORKLOADS[name]
        M, N, K = wl.gemm_shape
        S, U, hl, B, H = wl.s_local, wl.world, wl.local_heads, wl.batch, wl.heads
        sched = W.schedule_pairs(wl.schedule)
        xs = [device_normal(torch, dev, (B, S, wl.hidden), wl.x_std, wl.seed("x", c))
              for c in range(wl.calls)]
        w = device_normal(torch, dev, (N, K), 1.0 / np.sqrt(K), wl.seed("w"))
        wq_h, wk_h = W.norm_weights(wl)
        wq, wk = torch.from_numpy(wq_h).to(dev), torch.from_numpy(wk_h).to(dev)
        cs = torch.from_numpy(W.table(wl)).to(dev)
        sess = hx.qkvx_create(wl.hidden, H, 128, U, wl.layout, M, wl.num_slots)
        calls = [0]

        def fused():
            sess.forward(xs[calls[0] % len(xs)], w, wq, wk, cs, wl.rank, stream)
            calls[0] += 1

        for _ in range(3):
            fused()
        flops = 2.0 * M * N * K
        res = {"gemm_mnk": [M, N, K], "layout": wl.layout, "world": U,
               "schedule": list(wl.schedule), "fused_calls_cycled": wl.calls}
        for mode, ev in (("warm", None), ("cold", evict)):
            st = pct(launch_times(torch, fused, reps, stream, evict, ev))
            st["tflops"] = flops / (st["median_us"] * 1e-6) / 1e12
            st["frac"] = st["tflops"] / PEAK_BF16_TFLOPS
            res[f"fused_{mode}"] = st
        sess.close()
        # the pages' RoPE pairing (2i, 2i+1): the same launch with the other
        # epilogue branch, warm
        sess = hx.qkvx_create(wl.hidden, H, 128, U, wl.layout, M, wl.num_slots,
                              rope="interleaved")
        for _ in range(3):
            fused()
        st = pct(launch_times(torch, fused, reps, stream, evict, None))
        st["tflops"] = flops / (st["median_us"] * 1e-6) / 1e12
        st["frac"] = st["tflops"] / PEAK_BF16_TFLOPS
        res["fused_warm_interleaved_rope"] = st
        sess.close()
        del xs, w, sess
        torch.cuda.empty_cache()

        shape = (B, S, H, 128)
        if wl.pack_source == "fused384":
            base = device_normal(torch, dev, (B, S, H, 384), 1.0, wl.seed("qkv384"))
            q, k, v = base[..., :128], base[..., 128:256], base[..., 256:]
        else:
            q, k, v = (device_normal(torch, dev, shape, 1.0, wl.seed(t)) for t in "qkv")
        band = device_normal(torch, dev, (B, wl.s_global, hl, 128), 1.0, wl.seed("band"))
        srcs = [band[:, u * S:(u + 1) * S] for u in range(U)]
        mout = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        # every chunk's destinations stay allocated so that the whole schedule
        # can run as one group; chunk times are back to back (20 launches
        # between one pair of events), group times warm and after eviction
        chunks, fns, dsts = [], {"pack": [], "merge": []}, []
        for c, (off, cnt) in enumerate(sched):
            dst = [torch.empty(B, wl.s_global, cnt, 384, dtype=torch.bfloat16, device=dev)
                   for _ in range(U)]
            dsts.append(dst)
            cases = {
                "pack": (lambda c=c, dst=dst: hx.ulysses_pack_qkv_head_chunk(
                    q, k, v, world=U, schedule=wl.schedule, chunk=c, dst=dst,
                    row_offset=wl.rank * S, stream=stream), 2.0 * B * S * U * cnt * 384 * 2),
                "merge": (lambda c=c, off=off: hx.ulysses_merge_output_head_chunk(
                    srcs, world=U, local_heads=hl, schedule=wl.schedule, chunk=c, out=mout,
                    head_offset=off, stream=stream), 2.0 * B * S * U * cnt * 128 * 2),
            }
            row = {"heads": cnt}
            for kind, (fn, nbytes) in cases.items():
                us = back_to_back_us(torch, fn, stream)
                row[f"{kind}_bytes"] = nbytes
                row[f"{kind}_warm_us"] = us
                row[f"{kind}_warm_frac"] = nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS
                fns[kind].append(fn)
            chunks.append(row)
        res["chunks"] = chunks
        for kind in ("pack", "merge"):
            nbytes = sum(r[f"{kind}_bytes"] for r in chunks)
            group = lambda kind=kind: [f() for f in fns[kind]]
            for mode, us in (("warm", back_to_back_us(torch, group, stream)),
                             ("cold", cold_us(torch, group, stream, evict))):
                res[f"{kind}_{mode}_all_chunks"] = {
                    "us": us, "gbps": nbytes / (us * 1e-6) / 1e9,
                    "frac": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS}
        del dsts, fns
        out[name] = res
        del q, k, v, band, srcs, mout
        if wl.pack_source == "fused384":
            del base
        torch.cuda.empty_cache()
    del evict
    torch.cuda.empty_cache()
    return out


def output_side(hx, torch, wl, band, sched, dev, reps: int = 10):
    """Times the whole-band and output-side transforms of one rank on the same
    shard (outside the step): scatter_heads of a [B, S_local, H, 128] input,
    gather_heads of the [B, S_global, H_local, 128] band, the output sequence
    split of every chunk into contiguous staging, and exchange_chunks of the
    whole-band Q|K|V message (B*S_local*H_local*384 bf16 per peer).  Bytes are
    algorithmic: every element read once and written once."""
    S, U, hl, B = wl.s_local, wl.world, wl.local_heads, wl.batch
    stream = torch.cuda.current_stream()
    shard = device_normal(torch, dev, (B, S, wl.heads, 128), 1.0, wl.seed("shard"))
    scat = [torch.empty(B, wl.s_global, hl, 128, dtype=torch.bfloat16, device=dev)
            for _ in range(U)]
    gath = [torch.empty(B, S, wl.heads, 128, dtype=torch.bfloat16, device=dev) for _ in range(U)]
    staging = [torch.empty(U, B, S, cnt, 128, dtype=torch.bfloat16, device=dev)
               for _, cnt in sched]
    msg = B * S * hl * 384 * 2
    ex_x = device_normal(torch, dev, (U, msg // 2), 1.0, wl.seed("chunks")).view(torch.uint8)
    ex_out = [torch.empty(U, msg, dtype=torch.uint8, device=dev) for _ in range(U)]
    cases = {
        "scatter_heads": (lambda: hx.ulysses_scatter_heads(shard, world=U, dst=scat,
                                                           row_offset=wl.rank * S, stream=stream),
                          2.0 * shard.numel() * 2),
        "gather_heads": (lambda: hx.ulysses_gather_heads(band, world=U, dst=gath,
                                                         head_offset=wl.rank * hl, stream=stream),
                         2.0 * band.numel() * 2),
        "output_sequence_pack_all_chunks": (
            lambda: [hx.ulysses_pack_output_sequence_chunk(
                band[:, :, off:off + cnt], world=U, dst=[st[u] for u in range(U)], stream=stream)
                for (off, cnt), st in zip(sched, staging)],
            2.0 * band.numel() * 2),
        "exchange_chunks": (lambda: hx.ulysses_exchange_chunks(ex_x, world=U, rank=wl.rank,
                                                               dst=ex_out, stream=stream),
                            2.0 * U * msg),
    }
    out = {}
    for name, (fn, nbytes) in cases.items():
        us = back_to_back_us(torch, fn, stream, reps)
        gbps = nbytes / (us * 1e-6) / 1e9
        out[name] = {"us": us, "bytes": nbytes, "gbps": gbps, "frac": gbps / PEAK_HBM_GBPS}
    return out


def readiness(hx, torch, wl, x, w, wq, wk, cs, dev, reps: int = 5):
    """Forward with readiness words on one stream and a wait per destination on
    its own stream: when each destination's receive slot becomes readable,
    relative to the start of the call, and the call's own duration, beside the
    same call without publishing."""
    M = wl.tokens
    sess = hx.qkvx_create(wl.hidden, wl.heads, 128, wl.world, wl.layout, M, wl.num_slots)
    producer = torch.cuda.Stream()
    consumers = [torch.cuda.Stream() for _ in range(wl.world)]
    ev = lambda: torch.cuda.Event(enable_timing=True)
    plain = []
    for it in range(reps + 1):
        e0, e1 = ev(), ev()
        with torch.cuda.stream(producer):
            e0.record(producer)
            sess.forward(x, w, wq, wk, cs, wl.rank, producer)
            e1.record(producer)
        torch.cuda.synchronize()
        if it:
            plain.append(e0.elapsed_time(e1) * 1e3)
    sess.set_publish(True)
    fwd, ready = [], [[] for _ in range(wl.world)]
    for it in range(reps + 1):
        e0, e1 = ev(), ev()
        ed = [ev() for _ in range(wl.world)]
        with torch.cuda.stream(producer):
            e0.record(producer)
            sess.forward(x, w, wq, wk, cs, wl.rank, producer)
            e1.record(producer)
        for d, c in enumerate(consumers):
            c.wait_event(e0)            # the waits start with the call
            sess.wait_ready(d, stream=c)
            ed[d].record(c)
        torch.cuda.synchronize()
        if it:
            fwd.append(e0.elapsed_time(e1) * 1e3)
            for d in range(wl.world):
                ready[d].append(e0.elapsed_time(ed[d]) * 1e3)
    timeouts = sess.ready_state()[1]
    sess.close()
    return {"forward_us": float(np.mean(plain)), "publishing_forward_us": float(np.mean(fwd)),
            "dest_ready_us": [float(np.mean(r)) for r in ready], "wait_timeouts": timeouts}


def power_sample(torch, fn, seconds: float = 3.0, settle: float = 1.0):
    """Socket power and per-XCD shader clocks while ``fn`` runs back to back for
    about ``seconds``: ``amd-smi metric -p -c --csv`` polled from a thread (a
    child process per poll, 5 s limit each), keeping the polls that start after
    ``settle`` seconds (the power reading is an average that takes about a
    second to reach the steady state of a load).  Medians over the kept polls;
    None when the tool is missing or reports nothing."""
    import csv
    import io
    import shutil
    import statistics
    import subprocess
    import threading
    tool = shutil.which("amd-smi")
    if tool is None:
        return None
    rows, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            started = time.perf_counter() - t0
            try:
                r = subprocess.run([tool, "metric", "-p", "-c", "--csv"], capture_output=True,
                                   text=True, timeout=5)
            except (OSError, subprocess.SubprocessError):
                return
            if started >= settle:
                rows.append(r.stdout)
            stop.wait(0.2)

    warm_up(torch, fn)
    t0 = time.perf_counter()
    t = threading.Thread(target=poll)
    t.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    stop.set()
    t.join()
    vals = {}
    for text in rows:
        table = list(csv.reader(io.StringIO(text.strip())))
        if len(table) < 2:
            continue
        for h, v in zip(table[0], table[1]):
            keep = (h == "socket_power") or (h.startswith("gfx_") and h.endswith("_clk")
                                             and "min" not in h and "max" not in h)
            if keep:
                try:
                    vals.setdefault(h, []).append(float(v))
                except ValueError:
                    pass
    if not vals:
        return None
    clocks = [statistics.median(v) for h, v in sorted(vals.items()) if h.startswith("gfx_")]
    out = {"polls": len(rows), "tool": "amd-smi metric -p -c",
           "window_s": [settle, seconds]}
    if "socket_power" in vals:
        out["socket_power_w"] = statistics.median(vals["socket_power"])
    if clocks:
        out["xcd_clock_mhz"] = clocks
        out["xcd_clock_mhz_mean"] = statistics.mean(clocks)
    return out


def reference_gemm(torch, x, w, stream, reps: int = 10):
    """The vendor library's plain GEMM of the same shape, Y = X W^T in bf16
    (torch.mm, which calls hipBLASLt; no norm, RoPE or band store), timed per
    launch like the fused kernel, on the same inputs.  A reference point for the
    fused kernel's MFMA fraction under the same power limit, not part of the
    path."""
    xm = x.view(-1, x.shape[-1])
    wt = w.t()
    out = torch.empty(xm.shape[0], w.shape[0], dtype=torch.bfloat16, device=x.device)
    fn = lambda: torch.mm(xm, wt, out=out)
    ms = launch_times(torch, fn, reps, stream, out)
    M, K = xm.shape
    N = w.shape[0]
    st = pct(ms)
    st["tflops"] = 2.0 * M * N * K / (st["median_us"] * 1e-6) / 1e12
    st["frac"] = st["tflops"] / PEAK_BF16_TFLOPS
    st["what"] = "torch.mm (hipBLASLt) bf16 GEMM of the same M, N, K; output bf16, no epilogue"
    del out
    torch.cuda.empty_cache()
    return st


def head_chunk_pipeline(hx, torch, wl, q, k, v, sched, dev, reps: int = 5):
    """The pages' three-stream head-chunk schedule on one GPU: the input pack
    of chunk N+1, a stand-in consumer of chunk N and the output side of chunk
    N-1 overlap on three streams joined by events, against the same work on
    one stream.  Per chunk: pack Q|K|V of the band into a receive slot
    [B, S_global, hc, 384] (rows rank*S_local..); consumer: a bf16 matmul of
    the slot's q part by a [hc*128, hc*128] weight (a stand-in for attention,
    which is not part of this path) giving the output band [B, S_global, hc,
    128]; output side: its sequence split into the peers' received bands and
    the merge of the received band into the full output."""
    S, U, hl, B = wl.s_local, wl.world, wl.local_heads, wl.batch
    Sg = wl.s_global
    slots = {c: [torch.empty(B, Sg, c, 384, dtype=torch.bfloat16, device=dev) for _ in range(U)]
             for _, c in sched}
    wts = {c: torch.randn(c * 128, c * 128, device=dev).to(torch.bfloat16) / (c * 128) ** 0.5
           for _, c in sched}
    obands = {c: torch.empty(B, Sg, c, 128, dtype=torch.bfloat16, device=dev) for _, c in sched}
    received = {c: [torch.empty(B, S, U * c, 128, dtype=torch.bfloat16, device=dev)
                    for _ in range(U)] for _, c in sched}
    out = torch.empty(B, S, wl.heads, 128, dtype=torch.bfloat16, device=dev)

    def stage_in(i, st):
        c = sched[i][1]
        hx.ulysses_pack_qkv_head_chunk(q, k, v, world=U, schedule=wl.schedule, chunk=i,
                                       dst=slots[c], row_offset=wl.rank * S, stream=st)

    def stage_att(i, st):
        c = sched[i][1]
        with torch.cuda.stream(st):
            qp = slots[c][0][..., :128].reshape(B * Sg, c * 128)
            torch.matmul(qp.contiguous(), wts[c], out=obands[c].view(B * Sg, c * 128))

    def stage_out(i, st):
        off, c = sched[i]
        hx.ulysses_pack_output_sequence_chunk(obands[c], world=U, dst=received[c],
                                              head_offset=wl.rank * c, stream=st)
        hx.ulysses_merge_output_head_chunk([received[c][0][:, :, u * c:(u + 1) * c]
                                            for u in range(U)], world=U, local_heads=hl,
                                           schedule=wl.schedule, chunk=i, out=out, stream=st)

    main = torch.cuda.current_stream()
    s_in, s_att, s_out = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def sequential():
        for i in range(len(sched)):
            stage_in(i, main)
            stage_att(i, main)
            stage_out(i, main)

    def pipelined():
        start = torch.cuda.Event()
        start.record(main)
        for st in (s_in, s_att, s_out):
            st.wait_event(start)
        e_in = [torch.cuda.Event() for _ in sched]
        e_att = [torch.cuda.Event() for _ in sched]
        e_out = [torch.cuda.Event() for _ in sched]
        for i in range(len(sched)):
            stage_in(i, s_in)
            e_in[i].record(s_in)
            s_att.wait_event(e_in[i])
            stage_att(i, s_att)
            e_att[i].record(s_att)
            s_out.wait_event(e_att[i])
            stage_out(i, s_out)
            e_out[i].record(s_out)
        main.wait_event(e_out[-1])
        for st in (s_in, s_att):
            main.wait_stream(st)

    def serialized():
        # the same three streams and the same events, but every stage also waits
        # for the one before it: the cross-stream hand-offs without any overlap
        start = torch.cuda.Event()
        start.record(main)
        s_in.wait_event(start)
        last = None
        for i in range(len(sched)):
            for st, stage in ((s_in, stage_in), (s_att, stage_att), (s_out, stage_out)):
                if last is not None:
                    st.wait_event(last)
                stage(i, st)
                last = torch.cuda.Event()
                last.record(st)
        main.wait_event(last)

    res = {}
    for name, fn in (("sequential_us", sequential), ("pipelined_us", pipelined),
                     ("three_streams_serialized_us", serialized)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(main)
        for _ in range(reps):
            fn()
        e1.record(main)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1e3 / reps
    res["speedup"] = res["sequential_us"] / res["pipelined_us"]
    res["note"] = ("three_streams_serialized: the three streams with every stage waiting for the "
                   "previous one (cross-stream hand-offs, no overlap)")
    res["consumer"] = "bf16 matmul of the q band by a [hc*128, hc*128] weight (stand-in)"
    return res


def main():
    args = parse()
    world_env = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world_env != 1:
        print(json.dumps({"error": "this benchmark measures one GPU's share of the Ulysses "
                                   "exchange (peers simulated in local HBM); run it with --gpus 1"}))
        sys.exit(2)

    import torch
    import workloads as W
    import head_exchange_amd as hx

    hx.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = W.WORKLOADS[args.workload]
    M, N, K = wl.gemm_shape
    S, U, hl, B = wl.s_local, wl.world, wl.local_heads, wl.batch
    sched = W.schedule_pairs(wl.schedule)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    # ---- seeded inputs, resident in HBM ------------------------------------
    x_h = W.x_input(wl)
    w_h = W.w_qkv(wl)
    wq_h, wk_h = W.norm_weights(wl)
    cs_h = W.table(wl)
    qkv_h = W.pack_sources(wl)
    band_h = W.merge_band(wl)
    x, w = up(x_h), up(w_h)
    wq, wk = torch.from_numpy(wq_h).to(dev), torch.from_numpy(wk_h).to(dev)
    cs = torch.from_numpy(cs_h).to(dev)
    q, k, v = (up(a) for a in qkv_h)
    band = up(band_h)
    sess = hx.qkvx_create(wl.hidden, wl.heads, 128, U, wl.layout, M, wl.num_slots)
    pack_dst = [[torch.empty(B, wl.s_global, cnt, 384, dtype=torch.bfloat16, device=dev)
                 for _ in range(U)] for _, cnt in sched]
    merge_out = torch.empty(B, S, wl.heads, 128, dtype=torch.bfloat16, device=dev)
    merge_src = [band[:, u * S:(u + 1) * S] for u in range(U)]
    stream = torch.cuda.current_stream()

    def pack_group():
        for c in range(len(sched)):
            hx.ulysses_pack_qkv_head_chunk(q, k, v, world=U, schedule=wl.schedule, chunk=c,
                                           dst=pack_dst[c], row_offset=wl.rank * S, stream=stream)

    def merge_chunk(c):
        hx.ulysses_merge_output_head_chunk(merge_src, world=U, local_heads=hl,
                                           schedule=wl.schedule, chunk=c, out=merge_out,
                                           head_offset=sched[c][0], stream=stream)

    def merge_group():
        for c in range(len(sched)):
            merge_chunk(c)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        sess.forward(x, w, wq, wk, cs, wl.rank, stream)
        if ev is not None:
            ev[1].record(stream)
        pack_group()
        if ev is not None:
            ev[2].record(stream)
        merge_group()
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per = {name: [e[a].elapsed_time(e[a + 1]) for e in events]
           for a, name in enumerate(("fused", "pack_all_chunks", "merge_all_chunks"))}
    fused_ms, pack_ms, merge_ms = (float(np.mean(per[n])) for n in per)
    step_ms = wall * 1e3 / args.steps
    flops = 2.0 * M * N * K
    pack_bytes = sum(2.0 * B * S * U * cnt * 384 * 2 for _, cnt in sched)
    merge_bytes = sum(2.0 * B * S * U * cnt * 128 * 2 for _, cnt in sched)
    achieved = flops / (fused_ms * 1e-3) / 1e12
    traffic = read_traffic(args.workload)

    # The same pack and merge groups REPS times back to back between one pair
    # of events: the per-group time without the cost of the events themselves,
    # which the per-step figures above include (a pair of timing events around
    # one empty kernel measures about 6 us).
    REPS = 20

    def amortized_ms(group):
        return back_to_back_us(torch, group, stream, REPS) * 1e-3

    pack_rep_ms, merge_rep_ms = amortized_ms(pack_group), amortized_ms(merge_group)
    evict = torch.empty(EVICT_BYTES, dtype=torch.uint8, device=dev)
    evict.fill_(3)
    pack_cold_us = cold_us(torch, pack_group, stream, evict)
    merge_cold_us = cold_us(torch, merge_group, stream, evict)
    merge_chunk_bytes = [2.0 * B * S * U * cnt * 128 * 2 for _, cnt in sched]
    merge_chunk_cold = [cold_us(torch, lambda c=c: merge_chunk(c), stream, evict)
                        for c in range(len(sched))]
    merge_chunk_warm = [back_to_back_us(torch, lambda c=c: merge_chunk(c), stream)
                        for c in range(len(sched))]
    ceiling = copy_ceiling(torch, dev, stream, evict, wl)
    del evict
    torch.cuda.empty_cache()

    result = {
        "metric": "fused QKV+norm+RoPE+pack TFLOP/s and head-band pack/merge GB/s, 1 GPU",
        "value": flops / (step_ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "s_local": S, "s_global": wl.s_global,
                   "heads": wl.heads, "head_dim": 128, "hidden": wl.hidden, "world": U,
                   "rank": wl.rank, "layout": wl.layout, "schedule": list(wl.schedule),
                   "gemm_mnk": [M, N, K], "rope": "rotate_half", "rope_base": wl.rope_base,
                   "parallelism": f"ulysses shard of {U} (peers simulated in local HBM)"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic, "kernel": "fused_qkv_kernel",
                     "per_launch": f"2*M*N*K = {flops:.4g} FLOP"},
        "transport": {"pack_us": pack_ms * 1e3, "pack_gbps": pack_bytes / (pack_ms * 1e-3) / 1e9,
                      "pack_frac": pack_bytes / (pack_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                      "merge_us": merge_ms * 1e3,
                      "merge_gbps": merge_bytes / (merge_ms * 1e-3) / 1e9,
                      "merge_frac": merge_bytes / (merge_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                      "pack_bytes": pack_bytes, "merge_bytes": merge_bytes,
                      "peak_gbps": PEAK_HBM_GBPS,
                      "back_to_back": {
                          "groups": REPS,
                          "pack_us": pack_rep_ms * 1e3,
                          "pack_frac": pack_bytes / (pack_rep_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                          "merge_us": merge_rep_ms * 1e3,
                          "merge_frac": merge_bytes / (merge_rep_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS},
                      "cold": {
                          "note": "inputs from HBM: 10 x (read of a 1 GiB buffer, then the "
                                  "group) back to back minus 10 reads alone, per group; "
                                  "median of 5",
                          "merge_chunks": [
                              {"heads": cnt, "bytes": nb, "warm_us": wu,
                               "warm_frac": nb / (wu * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                               "cold_us": cu, "cold_frac": nb / (cu * 1e-6) / 1e9 / PEAK_HBM_GBPS}
                              for (_, cnt), nb, wu, cu in zip(sched, merge_chunk_bytes,
                                                              merge_chunk_warm, merge_chunk_cold)],
                          "pack_us": pack_cold_us,
                          "pack_frac": pack_bytes / (pack_cold_us * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                          "merge_us": merge_cold_us,
                          "merge_frac": merge_bytes / (merge_cold_us * 1e-6) / 1e9 / PEAK_HBM_GBPS},
                      "copy_ceiling": ceiling,
                      "timing_note": "pack_us and merge_us: per-step events around each group "
                                     "(a pair of events costs a few microseconds); back_to_back: "
                                     "20 groups between one pair of events"},
        "kernels_ms": {"fused": fused_ms, "pack_all_chunks": pack_ms, "merge_all_chunks": merge_ms},
        "kernels_pct": {n: pct(v) for n, v in per.items()},
    }
    if traffic is not None:
        result["roofline"]["traffic_from"] = profile_label(traffic_file(args.workload))
    counters = read_mfma_counters(args.workload)
    if counters:
        result["roofline"].update(counters)
        result["roofline"]["counters_from"] = profile_label(mfma_file(args.workload))
    result["reference_gemm"] = reference_gemm(torch, x, w, stream)
    xm, wt = x.view(-1, x.shape[-1]), w.t()
    for key, fn in (("power_under_fused_kernel",
                     lambda: sess.forward(x, w, wq, wk, cs, wl.rank, stream)),
                    ("power_under_reference_gemm", lambda: torch.mm(xm, wt))):
        if args.skip_power:
            result[key] = None
            continue
        try:
            result[key] = power_sample(torch, fn)
        except Exception as exc:          # the samples are context; never fail the bench on them
            result[key] = {"error": str(exc)[:200]}
    result["output_side"] = output_side(hx, torch, wl, band, sched, dev)
    result["readiness"] = readiness(hx, torch, wl, x, w, wq, wk, cs, dev)
    result["head_chunk_pipeline"] = head_chunk_pipeline(hx, torch, wl, q, k, v, sched, dev)
    if not args.skip_sweep:
        del q, k, v, band, pack_dst, merge_out, merge_src
        torch.cuda.empty_cache()
        result["sweep"] = sweep(hx, torch, W, dev)
    if not args.skip_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, x_h, w_h, wq_h, wk_h, cs_h, qkv_h, band_h,
                                              args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    sess.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
