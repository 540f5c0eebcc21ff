"""Benchmark of the exact-attention hot path on one MI355X.

One step = one pass of the whole path over resident synthetic inputs:
  * fused prefill  attn_fwd            on the long causal workload
    (bf16, b=1, s_q=s_k=16384, h=32, d=128), and
  * flash-decoding attn_fwd_splitkv + attn_combine on the decode workload
    (bf16, b=1, s_q=1, s_k=32768, h=16, d=128), split count from the
    compute-unit heuristic.
``value`` is the prefill throughput in TFLOP/s (algorithmic FLOPs: 4*d per
visible (query, key) pair) from the median of the per-launch HIP-event times of
the timed steps.  The decode figure (K+V bytes over the time of both decode
launches, taken between one pair of events, with L2 and the 256 MB MALL flushed
by a 512 MiB fill before each pass; median) is reported beside it.  Kernel
durations come from HIP events recorded on the stream the kernels run on.

Beside the rooflines the line carries what the device really sustains
(libattn_probe.so, include/attn_probe.h): the shader clock sampled during
back-to-back prefill launches, an MFMA loop on random bf16 operands (the
power-limited matrix-core ceiling) and a plain read of the decode's 268 MB
(the read ceiling flash-attention issue #1248 compares decoding with).

The backward pass (attn_bwd) is reported under "backward": the long causal
workload and issue #1335's two fp16 head-dim-16 workloads.  The float64 CPU
oracle is timed on the four smaller workloads in full and on a row sample of
the long one ("cpu_baseline").

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--only prefill|decode|backward]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
KERNEL_SOURCES = ["exact_attention_64_amd/csrc/attn_fwd.hip", "exact_attention_64_amd/csrc/attn_decode.hip",
                  "exact_attention_64_amd/csrc/attn_combine.hip", "exact_attention_64_amd/csrc/attn_small.hip",
                  "exact_attention_64_amd/csrc/attn_common.h", "exact_attention_64_amd/csrc/attn_tile.h",
                  "exact_attention_64_amd/csrc/attn_internal.h"]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters.md")
CPU_ROWS_PER_HEAD = 4096  # seeded query rows per head in the CPU-baseline sample (~12 s of oracle work)
FLUSH_BYTES = 512 << 20   # written before each decode pass: evicts L2 and the 256 MB MALL


def visible_pairs(w) -> int:
    if not w.causal:
        return w.b * w.h * w.s_q * w.s_k
    off = w.s_k - w.s_q
    per_head = sum(max(0, min(w.s_k, i + off + 1)) for i in range(w.s_q))
    return w.b * w.h * per_head


def flops(w) -> int:
    return 4 * w.d * visible_pairs(w)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kind: str):
    """HBM bytes per launch from the committed counter summary, if it matches the
    current kernel source; otherwise None."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    text = open(COUNTERS_FILE).read()
    m = re.search(r"kernel_hash:\s*(\w+)", text)
    if not m or m.group(1) != kernel_hash():
        return None
    m = re.search(kind + r"_hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    return float(m.group(1)) if m else None


def cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def device_facts(torch, dev):
    """Compute-unit count, name, L2 size and a measured copy bandwidth (1 GiB read
    + 1 GiB written by torch's copy kernel, best of four) for context."""
    props = torch.cuda.get_device_properties(dev)
    n = 1 << 30
    src = torch.empty(n // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    best = 1e30
    for _ in range(4):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    del src, dst
    return {"name": getattr(props, "gcnArchName", props.name), "compute_units": props.multi_processor_count,
            "l2_bytes": getattr(props, "L2_cache_size", None),
            "copy_gbs": round(2 * n / (best * 1e-3) / 1e9, 1)}


def cpu_baseline(w, budget_s: float = 12.0):
    """Time the float64 oracle on the machine's host cores: on a bounded sample of the
    prefill workload (whole heads' worth of seeded query rows until about
    ``budget_s`` seconds of work), and on the four smaller workloads in full
    (inputs generated and upcast outside the timed region)."""
    import numpy as np
    import oracle
    import workloads

    import torch

    q, k, v = workloads.make_workload(w)
    rows_all = workloads.sample_rows(w.s_q, CPU_ROWS_PER_HEAD, w.h, seed=42)
    done_flops = 0
    done_rows = 0
    heads = 0
    elapsed = 0.0
    off = w.s_k - w.s_q
    for hi in range(w.h):
        qh, kh, vh = (t[:, :, hi:hi + 1].to(torch.float64).numpy() for t in (q, k, v))
        t1 = time.perf_counter()
        oracle.attention_rows(qh, kh, vh, w.scale, w.causal, [rows_all[hi]])
        elapsed += time.perf_counter() - t1
        pairs = sum(min(w.s_k, r + off + 1) if w.causal else w.s_k for r in rows_all[hi])
        done_flops += 4 * w.d * pairs * w.b
        done_rows += len(rows_all[hi]) * w.b
        heads += 1
        if elapsed >= budget_s:
            break
    del q, k, v
    per_config = {}
    for name in ("C1", "C2", "C3", "C4"):
        wc = workloads.WORKLOADS[name]
        h64 = [t.to(torch.float64).numpy() for t in workloads.make_workload(wc)]
        t1 = time.perf_counter()
        oracle.attention(*h64, wc.scale, wc.causal)
        dt = time.perf_counter() - t1
        per_config[name] = dict(workload=wc.note, seconds=round(dt, 3), gflops=round(flops(wc) / dt / 1e9, 2),
                                full=True)
        del h64
    per_config["C5"] = dict(workload=w.note, seconds=round(elapsed, 3),
                            gflops=round(done_flops / elapsed / 1e9, 2), full=False,
                            extrapolated_full_s=round(elapsed * flops(w) / done_flops, 1))
    return {
        "value": round(done_flops / elapsed / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": cpu_threads(),
        "kind": "oracle",
        "sample": (f"float64 NumPy oracle, {done_rows} seeded query rows ({len(rows_all[0])} per head, "
                   f"{heads} of {w.h} heads) of the causal s=16384 workload, each over its full key "
                   f"prefix; {done_flops / 1e9:.1f} GFLOP in {elapsed:.2f} s on {cpu_model()}, "
                   f"{len(os.sched_getaffinity(0))} cores in the affinity mask; per_config holds the "
                   f"four smaller workloads timed in full"),
        "seconds": round(elapsed, 3),
        "extrapolated_full_s": round(elapsed * flops(w) / done_flops, 1),
        "per_config": per_config,
    }


def progress(msg: str) -> None:
    """One line on stderr as each part of the run ends (a long profiled run then shows progress)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def stats_ms(ts):
    """(median, min, mean) of a list of event times in ms."""
    ts = sorted(ts)
    return ts[len(ts) // 2], ts[0], sum(ts) / len(ts)


def shader_clock_mhz(torch, probe, run, launches, dev):
    """The shader clock while ``run`` (one prefill launch) repeats back to back.

    A one-wave probe on a second stream (default priority) reads the cycle counter
    (shader cycles) and the steady counter at its start and after most of the run.
    The steady counter's rate is taken from HIP events around the probe running
    alone for ~20 ms, which also gives the clock of a nearly idle device.
    Returns (MHz during the run, MHz of the lone probe, peak MHz)."""
    wall_attr_hz, peak_hz = probe.rates()
    out = torch.zeros(4, dtype=torch.int64, device=dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    probe.probe_clock(int(wall_attr_hz * 20e-3), dev, None, out)
    b.record()
    torch.cuda.synchronize()
    c0, c1, w0, w1 = out.tolist()
    secs = a.elapsed_time(b) * 1e-3
    wall_hz = (w1 - w0) / secs
    idle_mhz = (c1 - c0) / ((w1 - w0) / wall_hz) / 1e6
    run()
    torch.cuda.synchronize()
    a.record()
    run()
    b.record()
    torch.cuda.synchronize()
    one_s = a.elapsed_time(b) * 1e-3
    side = torch.cuda.Stream(dev)
    with torch.cuda.stream(side):
        probe.probe_clock(int(wall_hz * one_s * (launches - 2)), dev, side, out)
    for _ in range(launches):
        run()
    torch.cuda.synchronize()
    c0, c1, w0, w1 = out.tolist()
    mhz = (c1 - c0) / ((w1 - w0) / wall_hz) / 1e6
    return round(mhz, 1), round(idle_mhz, 1), round(peak_hz / 1e6, 1)


def mfma_ceiling(torch, probe, dev, E):
    """TFLOP/s of the register-only MFMA loop (8 waves per compute unit, random
    and constant bf16 operands), median of three calls each."""
    res = {}
    for key, rnd in (("random_operands", True), ("constant_operands", False)):
        ts = []
        for _ in range(3):
            a, b = E(), E()
            a.record()
            _, _, fl = probe.probe_mfma(2000, rnd, dev)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        med = sorted(ts)[1]
        res[key] = round(fl / (med * 1e-3) / 1e12, 1)
    return res


def read_ceiling(torch, probe, nbytes, flush, dev, E):
    """GB/s of a plain 16-byte nontemporal read of ``nbytes`` after a cache flush:
    the best of a few grid sizes, median of 10 reads each."""
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    best = None
    for grid in (256, 512, 1024, 2048):
        sink = torch.empty(grid, dtype=torch.int32, device=dev)
        ts = []
        for _ in range(10):
            flush.fill_(0.0)
            a, b = E(), E()
            a.record()
            probe.probe_read(buf, nbytes, grid=grid, sink=sink)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        med = stats_ms(ts)[0]
        if best is None or med < best[0]:
            best = (med, grid)
    del buf
    return {"bytes": nbytes, "us": round(best[0] * 1e3, 2), "gbs": round(nbytes / (best[0] * 1e-3) / 1e9, 1),
            "grid": best[1]}


def bench_backward(torch, ea, workloads, dev, E):
    """attn_bwd (delta, dQ, dK/dV kernels) on the long causal workload and on the
    two fp16 head-dim-16 workloads whose backward issue #1335 times.  Inputs,
    the forward's O and LSE, dO and every output resident in HBM; one event pair
    per call, caches flushed before each (outside the events); median, min and
    mean.  Algorithmic work: 10*d flops per visible (query, key) pair (five
    products of 2*d: S, dP, dV, dK, dQ; the dQ kernel's recomputation of S and dP
    is not counted)."""
    W = workloads.WORKLOADS
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    outd = {}
    for name, iters in (("C5", 5), ("C2", 50), ("C1", 50)):
        w = W[name]
        q, k, v = (t.to(dev) for t in workloads.make_workload(w))
        do = workloads.make_dout(w.b, w.s_q, w.h, w.d, w.dtype).to(dev)
        O, L = ea.attn_fwd(q, k, v, w.scale, w.causal)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty((w.b, w.h, w.s_q), dtype=torch.float32, device=dev)
        run = lambda: ea.attn_bwd(q, k, v, O, do, L, w.scale, w.causal, dq=dq, dk=dk, dv=dv,  # noqa: E731
                                  delta=delta)
        for _ in range(2):
            run()
        ts = []
        for _ in range(iters):
            flush.fill_(0.0)
            a, b = E(), E()
            a.record()
            run()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        ts.sort()
        med = ts[len(ts) // 2]
        fl = 10 * w.d * visible_pairs(w)
        outd[name] = dict(workload="backward of " + w.note, ms=round(med, 4), ms_min=round(ts[0], 4),
                          ms_mean=round(sum(ts) / len(ts), 4), calls=iters, flops_per_call=fl,
                          tflops=round(fl / (med * 1e-3) / 1e12, 2),
                          frac_mfma=round(fl / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4))
        if name == "C1":
            # host time per call at the tiny shape (issue #1335's subject): through
            # the binding, and through a plan with the arguments marshalled once
            plan = ea.BwdPlan(q, k, v, O, do, L, w.scale, w.causal, dq=dq, dk=dk, dv=dv, delta=delta)
            for key, fn in (("host_us_per_call", run), ("host_us_per_call_plan", plan)):
                fn()
                torch.cuda.synchronize()
                h0 = time.perf_counter()
                for _ in range(200):
                    fn()
                outd[name][key] = round((time.perf_counter() - h0) / 200 * 1e6, 2)
                torch.cuda.synchronize()
            del plan
        del q, k, v, do, O, L, dq, dk, dv, delta
    del flush
    return outd


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "backward"], default="all")
    ap.add_argument("--no-small", action="store_true", help="skip the per-workload side table")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the clock, MFMA-loop and read-ceiling probes and the split sweep "
                         "(counter runs that should see only the path's own kernels)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy five times (reference "
                         "kernel of known size for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path: heads (prefill) or the key sequence (decode) would be sharded "
              "across GPUs, see the design notes.", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_64_amd as ea
    from exact_attention_64_amd import _probe as probe
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calib:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": n, "launches": 5}), flush=True)
        return
    W = workloads.WORKLOADS
    wp, wd = W["C5"], W["C4"]
    do_p = args.only in ("all", "prefill")
    do_d = args.only in ("all", "decode")

    # ---- resident inputs and outputs
    if do_p:
        qp, kp, vp = (t.to(dev) for t in workloads.make_workload(wp))
        Op = torch.empty_like(qp)
        Lp = torch.empty((wp.b, wp.h, wp.s_q), dtype=torch.float32, device=dev)
    if do_d:
        qd, kd, vd = (t.to(dev) for t in workloads.make_workload(wd))
        n_splits = ea.attn_num_splits(wd.b, wd.h, wd.s_q, wd.s_k, wd.d)
        opart = torch.empty((n_splits, wd.b, wd.h, wd.s_q, wd.d), dtype=torch.float32, device=dev)
        lpart = torch.empty((n_splits, wd.b, wd.h, wd.s_q), dtype=torch.float32, device=dev)
        Od = torch.empty_like(qd)
        Ld = torch.empty((wd.b, wd.h, wd.s_q), dtype=torch.float32, device=dev)
        flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(evs):
        if do_p:
            evs[0].record()
            ea.attn_fwd(qp, kp, vp, wp.scale, wp.causal, out=Op, lse=Lp)
            evs[1].record()
        if do_d:
            # Cold caches for the decode pass: its 268 MB of K/V would otherwise
            # partly sit in the 256 MB MALL.  The fill runs before the events,
            # and one event pair brackets both decode launches.
            flush.fill_(0.0)
            evs[2].record()
            ea.attn_fwd_splitkv(qd, kd, vd, n_splits, wd.scale, False, o_part=opart, lse_part=lpart)
            ea.attn_combine(opart, lpart, qd.dtype, out=Od, lse=Ld)
            evs[4].record()

    for _ in range(args.warmup):
        step([E() for _ in range(5)])
    torch.cuda.synchronize()

    events = [[E() for _ in range(5)] for _ in range(args.steps)]
    t_start, t_end = E(), E()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        step(events[i])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = max(ms_total, wall * 1e3) / args.steps

    res = {}
    if do_p:
        p_med, p_min, p_mean = stats_ms([e[0].elapsed_time(e[1]) for e in events])
        res["prefill"] = dict(ms=p_med, ms_min=p_min, ms_mean=p_mean, tflops=flops(wp) / (p_med * 1e-3) / 1e12)
        progress(f"prefill timed: {p_med:.4f} ms median")
    if do_d:
        d_med, d_min, d_mean = stats_ms([e[2].elapsed_time(e[4]) for e in events])
        # Per-kernel durations of the two decode launches, from their own event
        # pairs in a separate loop after the timed steps (context only: the
        # decode figure is both launches between one pair of events).
        kev = [[E() for _ in range(4)] for _ in range(args.steps)]
        for e in kev:
            flush.fill_(0.0)
            e[0].record()
            ea.attn_fwd_splitkv(qd, kd, vd, n_splits, wd.scale, False, o_part=opart, lse_part=lpart)
            e[1].record()
            e[2].record()
            ea.attn_combine(opart, lpart, qd.dtype, out=Od, lse=Ld)
            e[3].record()
        torch.cuda.synchronize()
        s_ms = stats_ms([e[0].elapsed_time(e[1]) for e in kev])[0]
        c_ms = stats_ms([e[2].elapsed_time(e[3]) for e in kev])[0]
        kvb = 2 * 2 * wd.b * wd.s_k * wd.h * wd.d
        # Split-count sweep (issue #1248 compares hard-coded 2/4/8 splits with the
        # heuristic): split-KV + combine between one event pair, caches flushed,
        # median of 10 passes per count.
        sweep = {}
        for n in ([] if args.no_probes else sorted({8, 16, 32, 48, 64, 96, 128, n_splits})):
            op_n = torch.empty((n, wd.b, wd.h, wd.s_q, wd.d), dtype=torch.float32, device=dev)
            lp_n = torch.empty((n, wd.b, wd.h, wd.s_q), dtype=torch.float32, device=dev)
            ts = []
            for _ in range(10):
                flush.fill_(0.0)
                a, b = E(), E()
                a.record()
                ea.attn_fwd_splitkv(qd, kd, vd, n, wd.scale, False, o_part=op_n, lse_part=lp_n)
                ea.attn_combine(op_n, lp_n, qd.dtype, out=Od, lse=Ld)
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            sweep[str(n)] = round(stats_ms(ts)[0] * 1e3, 2)
            del op_n, lp_n
        res["decode"] = dict(ms=d_med, ms_min=d_min, ms_mean=d_mean, splitkv_ms=s_ms, combine_ms=c_ms,
                             gbs=kvb / (d_med * 1e-3) / 1e9, kv_bytes=kvb, splits=n_splits, sweep=sweep,
                             read=None if args.no_probes else read_ceiling(torch, probe, kvb, flush, dev, E))
        progress(f"decode timed: {d_med * 1e3:.2f} us median")

    # ---- what the device sustains: shader clock during back-to-back prefill
    # launches, and the power-limited MFMA ceiling of a register-only loop
    if do_p and not args.no_probes:
        run_p = lambda: ea.attn_fwd(qp, kp, vp, wp.scale, wp.causal, out=Op, lse=Lp)  # noqa: E731
        res["prefill"]["sclk"] = shader_clock_mhz(torch, probe, run_p, 12, dev)
        res["prefill"]["mfma_ceiling"] = mfma_ceiling(torch, probe, dev, E)

    # ---- side table: the three smaller prefill workloads.  Event time per launch
    # (median, min, mean over 200 launches for C1/C2, 20 for C3, caches flushed
    # before each), and the host time of one call through the binding.
    side = {}
    if not args.no_small and args.only == "all":
        flush_s = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        for name, iters in (("C1", 200), ("C2", 200), ("C3", 20)):
            w = W[name]
            q, k, v = (t.to(dev) for t in workloads.make_workload(w))
            O = torch.empty_like(q)
            L = torch.empty((w.b, w.h, w.s_q), dtype=torch.float32, device=dev)
            for _ in range(3):
                ea.attn_fwd(q, k, v, w.scale, w.causal, out=O, lse=L)
            ts = []
            for _ in range(iters):
                flush_s.fill_(0.0)
                a, b = E(), E()
                a.record()
                ea.attn_fwd(q, k, v, w.scale, w.causal, out=O, lse=L)
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            torch.cuda.synchronize()
            h0 = time.perf_counter()
            for _ in range(iters):
                ea.attn_fwd(q, k, v, w.scale, w.causal, out=O, lse=L)
            host_us = (time.perf_counter() - h0) / iters * 1e6
            torch.cuda.synchronize()
            # the same call through a plan (arguments marshalled once)
            plan = ea.FwdPlan(q, k, v, w.scale, w.causal, out=O, lse=L)
            plan()
            torch.cuda.synchronize()
            h0 = time.perf_counter()
            for _ in range(iters):
                plan()
            plan_host_us = (time.perf_counter() - h0) / iters * 1e6
            torch.cuda.synchronize()
            ts.sort()
            med = ts[len(ts) // 2]
            io = 2 * w.b * w.h * w.d * (2 * w.s_q + 2 * w.s_k) + 4 * w.b * w.h * w.s_q
            side[name] = dict(workload=w.note, us=round(med * 1e3, 2), us_min=round(ts[0] * 1e3, 2),
                              us_mean=round(sum(ts) / len(ts) * 1e3, 2), launches=iters,
                              host_us_per_call=round(host_us, 2),
                              host_us_per_call_plan=round(plan_host_us, 2),
                              tflops=round(flops(w) / (med * 1e-3) / 1e12, 2),
                              io_gbs=round(io / (med * 1e-3) / 1e9, 1),
                              frac_mfma=round(flops(w) / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4))
            del q, k, v, O, L
        # The tiny workload through a HIP graph: 16 calls captured once, the graph
        # replayed 50 times between one event pair; device time and host time per call.
        w = W["C1"]
        q, k, v = (t.to(dev) for t in workloads.make_workload(w))
        O = torch.empty_like(q)
        L = torch.empty((w.b, w.h, w.s_q), dtype=torch.float32, device=dev)
        ea.attn_fwd(q, k, v, w.scale, w.causal, out=O, lse=L)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(16):
                ea.attn_fwd(q, k, v, w.scale, w.causal, out=O, lse=L)
        g.replay()
        torch.cuda.synchronize()
        a, b = E(), E()
        h0 = time.perf_counter()
        a.record()
        for _ in range(50):
            g.replay()
        b.record()
        host_us = (time.perf_counter() - h0) / (50 * 16) * 1e6
        torch.cuda.synchronize()
        dev_us = a.elapsed_time(b) / (50 * 16) * 1e3
        side["C1_graph"] = dict(workload=w.note + ", 16 calls per HIP graph replay", us_per_call=round(dev_us, 2),
                                host_us_per_call=round(host_us, 2), calls=50 * 16)
        del g, q, k, v, O, L
        # Multi-token decode with shared K/V heads (b=8, 48 query heads over 8 K/V
        # heads, a 4096-key cache, 1 or 4 new tokens): split-KV + combine with the
        # heuristic's split count, over the contiguous cache and over a paged one
        # (64-key blocks, scattered), one event pair around both launches after a
        # cache flush, median of 20 passes.
        for s_q in (1, 4):
            q, k, v = (t.to(dev) for t in workloads.make_qkv(8, s_q, 4096, 48, 128, "bf16", seed=19, h_kv=8))
            _, kc, vc, table, sl = (t.to(dev) for t in workloads.make_paged(8, s_q, 48, 128, "bf16", [4096] * 8,
                                                                             64, h_kv=8, seed=19))
            kvb = 2 * k.numel() * 2
            for kind in ("contiguous", "paged"):
                if kind == "contiguous":
                    n = ea.attn_num_splits(8, 48, s_q, 4096, 128, h_kv=8)
                    run = lambda: ea.attn_fwd_splitkv(q, k, v, n, None, True, o_part=op, lse_part=lp)  # noqa: E731
                else:
                    n = ea.attn_num_splits_paged(8, 48, s_q, 4096, 128, h_kv=8)
                    run = lambda: ea.attn_fwd_splitkv_paged(q, kc, vc, table, sl, n, 4096, None, True,  # noqa: E731
                                                            o_part=op, lse_part=lp)
                op = torch.empty((n, 8, 48, s_q, 128), dtype=torch.float32, device=dev)
                lp = torch.empty((n, 8, 48, s_q), dtype=torch.float32, device=dev)
                O = torch.empty_like(q)
                run()
                ts = []
                for _ in range(20):
                    flush_s.fill_(0.0)
                    a, b = E(), E()
                    a.record()
                    run()
                    ea.attn_combine(op, lp, q.dtype, out=O, lse=None, return_lse=False)
                    b.record()
                    torch.cuda.synchronize()
                    ts.append(a.elapsed_time(b))
                med, mn, mean = stats_ms(ts)
                side[f"gqa_decode_{kind}_s_q{s_q}"] = dict(
                    workload=f"bf16 causal b=8 s_q={s_q} s_k=4096 h=48 h_kv=8 d=128, {kind} K/V"
                             + (" (64-key blocks)" if kind == "paged" else "") + ", split-KV + combine",
                    us=round(med * 1e3, 2), us_min=round(mn * 1e3, 2), us_mean=round(mean * 1e3, 2), splits=n,
                    kv_gbs=round(kvb / (med * 1e-3) / 1e9, 1),
                    frac_hbm=round(kvb / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
            del q, k, v, kc, vc, table, sl, op, lp, O
        del flush_s
        progress("smaller workloads timed")

    out = {
        "metric": "attn fwd TFLOP/s (prefill) & decode K/V GB/s, % of MI355X MFMA/HBM peak",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q, k, v rounded to bf16 on the host)",
    }
    if do_p:
        p = res["prefill"]
        out.update(value=round(p["tflops"], 2), unit="TFLOP/s")
        out["config"] = {
            "workload": "causal prefill bf16 b=1 s_q=s_k=16384 h=32 d=128 (attn_fwd)"
                        + (" + split-KV decode bf16 b=1 s_q=1 s_k=32768 h=16 d=128 "
                           "(attn_fwd_splitkv + attn_combine)" if do_d else ""),
            "b": wp.b, "s_q": wp.s_q, "s_k": wp.s_k, "h": wp.h, "d": wp.d, "causal": True,
        }
        sclk, idle_mhz, peak_mhz = p.get("sclk", (None, None, None))
        ceil = p.get("mfma_ceiling", {"random_operands": None, "constant_operands": None})
        out["roofline"] = {
            "bound": "mfma", "achieved": round(p["tflops"], 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(p["tflops"] / PEAK_BF16_TFLOPS, 4),
            "traffic": read_traffic("prefill"),
            "kernel": "fwdp_kernel (attn_fwd, d >= 64 prefill)",
            "launch_ms_median": round(p["ms"], 4), "launch_ms_min": round(p["ms_min"], 4),
            "launch_ms_mean": round(p["ms_mean"], 4), "launches": args.steps,
            "flops_per_launch": flops(wp),
            "sclk_mhz": sclk, "sclk_idle_probe_mhz": idle_mhz, "sclk_peak_mhz": peak_mhz,
            "frac_at_sclk": round(p["tflops"] / (PEAK_BF16_TFLOPS * sclk / peak_mhz), 4) if sclk else None,
            "mfma_loop_random_tflops": ceil["random_operands"],
            "mfma_loop_constant_tflops": ceil["constant_operands"],
            "frac_of_random_mfma_loop": (round(p["tflops"] / ceil["random_operands"], 4)
                                         if ceil["random_operands"] else None),
        }
    if do_d:
        dd = res["decode"]
        rd = dd["read"]
        dec = {
            "value": round(dd["gbs"], 1), "unit": "GB/s", "us": round(dd["ms"] * 1e3, 2),
            "us_min": round(dd["ms_min"] * 1e3, 2), "us_mean": round(dd["ms_mean"] * 1e3, 2),
            "splitkv_us": round(dd["splitkv_ms"] * 1e3, 2), "combine_us": round(dd["combine_ms"] * 1e3, 2),
            "splits": dd["splits"], "frac_hbm": round(dd["gbs"] / PEAK_HBM_GBS, 4),
            "read_ceiling": rd, "frac_of_read_ceiling": round(dd["gbs"] / rd["gbs"], 4) if rd else None,
            "split_sweep_us": dd["sweep"],
        }
        rdl = {
            "bound": "hbm", "achieved": round(dd["gbs"], 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(dd["gbs"] / PEAK_HBM_GBS, 4),
            "traffic": read_traffic("decode"),
            "kernel": "decode_kernel + combine_kernel (attn_fwd_splitkv + attn_combine, s_q = 1)",
            "launch_us_median": round(dd["ms"] * 1e3, 2), "bytes_per_launch": dd["kv_bytes"],
            "splitkv_only_gbs": round(dd["kv_bytes"] / (dd["splitkv_ms"] * 1e-3) / 1e9, 1),
        }
        if do_p:
            out["decode"] = dec
            out["roofline_decode"] = rdl
        else:
            out.update(value=dec["value"], unit="GB/s")
            out["config"] = {"workload": "split-KV decode bf16 b=1 s_q=1 s_k=32768 h=16 d=128",
                             "b": wd.b, "s_q": wd.s_q, "s_k": wd.s_k, "h": wd.h, "d": wd.d}
            out["decode"] = dec
            out["roofline"] = rdl
    if side:
        out["other_workloads"] = side
    if args.only in ("all", "backward") and not args.no_small:
        out["backward"] = bench_backward(torch, ea, workloads, dev, E)
        progress("backward timed")
        if args.only == "backward":
            bc5 = out["backward"]["C5"]
            out.update(value=bc5["tflops"], unit="TFLOP/s", config={
                "workload": "backward (attn_bwd) of the causal prefill bf16 b=1 s_q=s_k=16384 h=32 d=128",
                "b": wp.b, "s_q": wp.s_q, "s_k": wp.s_k, "h": wp.h, "d": wp.d, "causal": True})
    if args.only == "all" and not args.no_small:
        out["device"] = device_facts(torch, dev)
    if not args.no_cpu and do_p:
        out["cpu_baseline"] = cpu_baseline(wp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
