"""Throughput of the window put/get collectives on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-rows] [--no-cpu]

A step is one sum-AllReduce of 8 virtual ranks x 64 Mi bf16 elements each
(fp32 accumulation in fixed rank order, bf16 output): reduce-scatter by gets
and all-gather by puts with a SignalInc per (owner, receiver), receivers
waiting in-kernel -- the whole hot path, one kernel launch. Inputs are
seeded normal(0, 1) values already resident in HBM when the timed region
starts. The metric is achieved HBM GB/s over the algorithmic bytes
2 * R * N * 2 (every input byte read once, every output byte written once).

Printed: one JSON line with the metric, the roofline of the AllReduce kernel
(its algorithmic bytes over its event-timed duration, against the 8 TB/s
HBM3E peak), the CPU oracle timed on a bounded sample, and -- unless
--no-rows -- the other workloads (1 GiB put and get, a 256 B signal
ping-pong, AllReduce fp32 R=4,
AlltoAll by compute units, in barrier sessions and by the copy engines,
dispatch, combine, their per-rank-dedup forms, AllGather by compute units
and by the copy engines, ring exchange with strong and weak signals) each
measured the same way, with the 256 MiB Infinity Cache flushed before every
timed repetition, and again back to back (no flush) as the headline is.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "achieved HBM GB/s (and % of peak) for R-rank AllReduce/AlltoAll/dispatch"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "k_allreduce": "allreduce.hip", "k_alltoall": "alltoall.hip", "k_allgather": "allgather.hip",
    "k_dispatch": "dispatch.hip", "k_combine": "combine.hip", "k_ring": "ring.hip",
    "k_alltoall_sessions": "sessions.hip", "k_dispatch_dedup": "dispatch.hip", "k_combine_dedup": "combine.hip",
    "k_ring_weak": "ring.hip", "k_put": "comm.hip", "k_pingpong": "pingpong.hip",
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(kernel: str) -> str:
    """Hash of a kernel's source and the shared device header (to age traffic figures)."""
    h = hashlib.sha256()
    files = [os.path.join("collective_window_put_amd", "csrc", f) for f in (KERNEL_SOURCES[kernel], "vr_device.hpp")]
    if kernel == "k_alltoall_sessions":
        files.append(os.path.join("include", "vrcomm_device.hpp"))
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter runs, if they match this source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(f"{kernel}:{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


class Bench:
    def __init__(self):
        import torch
        import collective_window_put_amd as vr
        self.torch, self.vr = torch, vr
        torch.cuda.set_device(0)
        self.stream = torch.cuda.current_stream()
        self.flush_buf = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")

    def slices(self, R: int, nbytes: int, arrays=None, fill=None):
        torch = self.torch
        a = self.vr.VR_WIN_REQUIRED_ALIGNMENT
        stride = (nbytes + a - 1) // a * a
        slab = torch.empty(R * stride + a, dtype=torch.uint8, device="cuda")
        s = (-slab.data_ptr()) % a
        views = [slab[s + r * stride: s + r * stride + nbytes] for r in range(R)]
        if arrays is not None:
            for v, x in zip(views, arrays):
                v.copy_(torch.from_numpy(np.ascontiguousarray(x).reshape(-1).view(np.uint8)))
        elif fill is not None:
            slab.fill_(fill)
        return slab, views

    def flush_cache(self):
        # Reading 1 GiB evicts the 256 MiB Infinity Cache and the L2s without
        # leaving dirty lines behind (a write flush would leave up to 256 MiB
        # of dirty lines to be written back inside the next timed kernel).
        self.flush_buf.view(self.torch.int64).sum()

    def warm(self, fn, n: int = 5):
        """Untimed warm-up calls before a row's timed repetitions."""
        for _ in range(n):
            fn()

    def timed(self, fn, reps: int, flush: bool):
        """Per-repetition durations (ms) from events recorded on the launch stream.

        With flush, the caches are evicted by a read before every repetition,
        and the result also carries `b2b_ms`: the same call timed `reps`
        times back to back between two events (the headline's timing mode).
        The two bracket the HBM-bound time from both sides: after a read
        flush the Infinity Cache is clean, so up to 256 MiB of a call's last
        writes can still sit there when the timer stops; back to back, each
        call pays for the write-back of the previous call's dirty lines, but
        may find some of its inputs still cached."""
        torch = self.torch
        out = Times()
        for _ in range(reps):
            if flush:
                self.flush_cache()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            fn()
            e1.record(self.stream)
            e1.synchronize()
            out.append(e0.elapsed_time(e1))
        if flush:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            fn()
            e0.record(self.stream)
            for _ in range(reps):
                fn()
            e1.record(self.stream)
            e1.synchronize()
            out.b2b_ms = e0.elapsed_time(e1) / reps
        return out


class Times(list):
    """Durations (ms) of the flushed repetitions; b2b_ms: back-to-back mean."""
    b2b_ms = None


def row_entry(name, bytes_alg, times_ms, kernel, workload, extra=None):
    med = float(np.median(times_ms))
    gbs = bytes_alg / (med * 1e-3) / 1e9
    d = {"algorithmic_bytes": int(bytes_alg), "median_ms": round(med, 5), "min_ms": round(float(np.min(times_ms)), 5),
         "GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "kernel": kernel,
         "traffic_bytes_per_launch": measured_traffic(kernel, workload) if kernel in KERNEL_SOURCES else None}
    b2b = getattr(times_ms, "b2b_ms", None)
    if b2b:
        d["back_to_back_ms"] = round(b2b, 5)
        d["back_to_back_GBps"] = round(bytes_alg / (b2b * 1e-3) / 1e9, 1)
    if extra:
        d.update(extra)
    log(f"{name}: {gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of peak), median {med:.4f} ms"
        + (f"; back to back {d['back_to_back_GBps']:.1f} GB/s, {b2b:.4f} ms" if b2b else ""))
    return d


# ---- the headline workload -------------------------------------------------------------------
def run_allreduce_headline(b: Bench, steps: int, warmup: int):
    import workloads as W
    vr = b.vr
    c = W.CONFIGS["allreduce_bf16_r8_64Mi"]
    R, N = c["ranks"], c["count"]
    log(f"generating AllReduce inputs R={R} N={N} bf16")
    xs = W.allreduce_bf16_inputs(R, N, seed=c["seed"])
    comm = vr.vr_comm_create(R, signal_count=4)
    s_slab, sv = b.slices(R, N * 2, arrays=xs)
    r_slab, rv = b.slices(R, N * 2, fill=0)
    sw = vr.vr_window_register(comm, [v.data_ptr() for v in sv], N * 2)
    rw = vr.vr_window_register(comm, [v.data_ptr() for v in rv], N * 2)
    stream = b.stream.cuda_stream

    def step():
        vr.vr_allreduce(comm, sw, 0, rw, 0, N, vr.VR_DT_BF16, sig=0, stream=stream)

    for _ in range(warmup):
        step()
    b.torch.cuda.synchronize()
    # timed region: K back-to-back steps between two events on the launch
    # stream (an event between every two steps would stretch each step by
    # ~8 us: measured 0.408 against 0.398 ms per step)
    e0 = b.torch.cuda.Event(enable_timing=True)
    e1 = b.torch.cuda.Event(enable_timing=True)
    b.torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(b.stream)
    for _ in range(steps):
        step()
    e1.record(b.stream)
    b.torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [e0.elapsed_time(e1) / steps]
    # the same step timed cold as well: 20 repetitions, each after a 1 GiB
    # read that evicts the caches, events around each (untimed by the headline)
    flushed = b.timed(step, 20, flush=True)
    code, bits = vr.vr_comm_get_async_error(comm)
    if code != vr.VR_OK:
        raise RuntimeError(f"device error during the AllReduce: {vr.vr_error_string(code)} bits={bits:#x}")
    # spot-check the last result against the fixed rank-order sum on a sample of elements
    idx = np.random.default_rng(0).integers(0, N, 4096)
    acc = (xs[0][idx].astype(np.uint32) << 16).view(np.float32)
    for r in range(1, R):
        acc = acc + (xs[r][idx].astype(np.uint32) << 16).view(np.float32)
    u = acc.view(np.uint32)
    exp = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    for d in (0, R - 1):
        got = rv[d].view(b.torch.int16).cpu().numpy().view(np.uint16)[idx]
        if not np.array_equal(got, exp):
            raise RuntimeError(f"AllReduce result mismatch on rank {d}")
    bytes_alg = 2 * R * N * 2
    ms_per_step = wall * 1e3 / steps
    vr.vr_window_deregister(comm, sw)
    vr.vr_window_deregister(comm, rw)
    vr.vr_comm_destroy(comm)
    del s_slab, r_slab
    return dict(xs=xs, R=R, N=N, bytes_alg=bytes_alg, ms_per_step=ms_per_step, kern_ms=kern_ms,
                flushed_ms=[float(t) for t in flushed])


# ---- the dispatch's phase timeline -----------------------------------------------------------------
PHASES = {"count": ["start", "histograms stored", "count row published (last block of a source)"],
          "put": ["start", "entries ranked, token-row loads issued", "count signal seen",
                  "count rows loaded, offsets computed", "source tags stored", "row stores issued",
                  "row stores complete", "row signals applied (last block of a source)"],
          "receiver": ["start", "count signal seen", "row signal seen"]}


def dispatch_phases(b: Bench, reps: int, dedup: bool = False) -> str:
    """Markdown timeline of the dispatch workload (8 ranks x 4096 tokens of
    512 B, top-8 of 256 Zipf(1.1) experts): every workgroup's phase
    timestamps (vr_comm_set_trace, device real-time clock) over `reps`
    launches, each after a 1 GiB read flush; times are from the first
    workgroup's start in the same launch. Per phase: the median over launches
    of the median, the earliest and the latest workgroup."""
    import workloads as W
    vr, stream, torch = b.vr, b.stream.cuda_stream, b.torch
    c = W.CONFIGS["dispatch_r8_t4096_e256_k8"]
    R, T, H, E, K = c["ranks"], c["tokens"], c["hidden"], c["experts"], c["topk"]
    topk, x = W.dispatch_inputs(R, T, H, E, K, c["zipf_s"], seed=c["seed"])
    rb = H * 2
    cap = R * T * (1 if dedup else min(K, E // R))
    comm = comm_for(vr, R, signal_count=4)
    s1, xv = b.slices(R, T * rb, arrays=[x[r] for r in range(R)])
    r1, rv = b.slices(R, cap * rb, fill=0)
    xw = vr.vr_window_register(comm, [v.data_ptr() for v in xv], T * rb)
    rw = vr.vr_window_register(comm, [v.data_ptr() for v in rv], cap * rb)
    tk = torch.from_numpy(topk).cuda()
    counts = torch.zeros(R, E // R, dtype=torch.int32, device="cuda")
    src = torch.zeros(R, cap, dtype=torch.int32, device="cuda")
    ex = torch.zeros(R, cap, K, dtype=torch.int32, device="cuda")
    nb1 = (T + 255) // 256
    ncount, nput = R * nb1, R * 4 * nb1
    grid = ncount + nput + R
    stamps = torch.zeros(grid * 8, dtype=torch.int64, device="cuda")

    def f():
        if dedup:
            vr.vr_dispatch_dedup(comm, xw, 0, rb, tk, T, K, E, rw, 0, cap, counts, src, ex, None, 0, 1, stream=stream)
        else:
            vr.vr_dispatch(comm, xw, 0, rb, tk, T, K, E, rw, 0, cap, counts, src, None, 0, 1, stream=stream)

    b.warm(f)
    vr.vr_comm_set_trace(comm, stamps)
    per = {k: [[] for _ in v] for k, v in PHASES.items()}
    events = []
    for _ in range(reps):
        stamps.zero_()
        b.flush_cache()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(b.stream)
        f()
        e1.record(b.stream)
        e1.synchronize()
        events.append(e0.elapsed_time(e1))
        st = stamps.view(grid, 8).cpu().numpy().astype(np.int64)
        t0 = st[:, 0][st[:, 0] > 0].min()
        kinds = {"count": st[:ncount], "put": st[ncount:ncount + nput], "receiver": st[ncount + nput:]}
        for k, arr in kinds.items():
            for ph in range(len(PHASES[k])):
                col = arr[:, ph]
                col = (col[col > 0] - t0) / 1e3  # us
                if col.size:
                    per[k][ph].append((np.median(col), col.min(), col.max(), col.size))
    vr.vr_comm_set_trace(comm, None)
    code, bits = vr.vr_comm_get_async_error(comm)
    if code != vr.VR_OK:
        raise RuntimeError(f"device error during the traced dispatch: {vr.vr_error_string(code)} bits={bits:#x}")
    vr.vr_window_deregister(comm, xw)
    vr.vr_window_deregister(comm, rw)
    vr.vr_comm_destroy(comm)
    lines = [f"{'Per-rank (dedup) dispatch' if dedup else 'Dispatch'}: R={R}, T={T}, {rb} B rows, E={E}, K={K}, "
             f"{reps} launches, each after a 1 GiB read flush; event time per launch (median) "
             f"{np.median(events) * 1e3:.1f} us", "",
             "| Workgroups | Phase | median WG (us) | first WG (us) | last WG (us) | WGs |",
             "|---|---|---|---|---|---|"]
    for k, names in PHASES.items():
        for ph, name in enumerate(names):
            v = per[k][ph]
            if not v:
                continue
            med = np.median([q[0] for q in v])
            lo = np.median([q[1] for q in v])
            hi = np.median([q[2] for q in v])
            n = int(np.median([q[3] for q in v]))
            lines.append(f"| {k} | {ph} {name} | {med:.2f} | {lo:.2f} | {hi:.2f} | {n} |")
    return "\n".join(lines)


# ---- the other workloads ------------------------------------------------------------------------
ROW_NAMES = ("put_get", "pingpong", "allreduce_f32", "alltoall", "alltoall_sessions", "alltoall_ce", "dispatch", "combine", "dedup",
             "allgather", "allgather_ce", "ring", "ring_weak")


def run_rows(b: Bench, reps: int = 10, only=ROW_NAMES):
    rows = {}
    if "put_get" in only:
        run_put_get_rows(b, reps, rows)
    if "pingpong" in only:
        run_pingpong_rows(b, reps, rows)
    # AllReduce fp32, R=4, 1 Mi elements (the worked-example shape)
    if "allreduce_f32" in only:
        run_allreduce_f32_row(b, reps, rows)
    if "alltoall" in only:
        run_alltoall_row(b, reps, rows)
    if "alltoall_sessions" in only:
        run_alltoall_row(b, reps, rows, sessions=True)
    if "alltoall_ce" in only:
        run_alltoall_row(b, reps, rows, copy_engine=True)
    if "dispatch" in only:
        run_dispatch_row(b, reps, rows)
    if "combine" in only:
        run_combine_row(b, reps, rows)
    if "dedup" in only:
        run_dedup_rows(b, reps, rows)
    if "allgather" in only:
        run_allgather_row(b, reps, rows)
    if "allgather_ce" in only:
        run_allgather_row(b, reps, rows, copy_engine=True)
    if "ring" in only:
        run_ring_row(b, reps, rows)
    if "ring_weak" in only:
        run_ring_row(b, reps, rows, weak=True)
    return rows


def comm_for(vr, R, **kw):
    return vr.vr_comm_create(R, **kw)


def run_allreduce_f32_row(b, reps, rows):
    import workloads as W
    vr, stream = b.vr, b.stream.cuda_stream
    c = W.CONFIGS["allreduce_f32_r4_1Mi"]
    R, N = c["ranks"], c["count"]
    xs = W.allreduce_f32_inputs(R, N, run="B", seed=c["seed"])
    comm = comm_for(vr, R, signal_count=2)
    s1, sv = b.slices(R, N * 4, arrays=xs)
    r1, rv = b.slices(R, N * 4, fill=0)
    sw = vr.vr_window_register(comm, [v.data_ptr() for v in sv], N * 4)
    rw = vr.vr_window_register(comm, [v.data_ptr() for v in rv], N * 4)
    f = lambda: vr.vr_allreduce(comm, sw, 0, rw, 0, N, vr.VR_DT_F32, sig=0, stream=stream)  # noqa: E731
    b.warm(f)
    rows["allreduce_f32_r4_1Mi"] = row_entry("AllReduce fp32 R=4 N=1Mi", 2 * R * N * 4, b.timed(f, reps, True),
                                             "k_allreduce", "allreduce_f32_r4_1Mi")
    vr.vr_window_deregister(comm, sw)
    vr.vr_window_deregister(comm, rw)
    vr.vr_comm_destroy(comm)
    del s1, r1



def run_alltoall_row(b, reps, rows, sessions=False, copy_engine=False):
    import workloads as W
    vr, stream = b.vr, b.stream.cuda_stream
    c = W.CONFIGS["alltoall_r8_4MiB"]
    R, B = c["ranks"], c["block_bytes"]
    sends = W.alltoall_inputs(R, B, seed=c["seed"])
    comm = comm_for(vr, R, signal_count=2, barrier_count=1)
    s1, sv = b.slices(R, R * B, arrays=sends)
    r1, rv = b.slices(R, R * B, fill=0)
    sw = vr.vr_window_register(comm, [v.data_ptr() for v in sv], R * B)
    rw = vr.vr_window_register(comm, [v.data_ptr() for v in rv], R * B)
    if sessions:  # the same exchange inside entry and exit barrier-session syncs
        f = lambda: vr.vr_alltoall_sessions(comm, sw, 0, rw, 0, B, sig=0, barrier_index=0,  # noqa: E731
                                            stream=stream)
        name, kernel, label = "alltoall_sessions_r8_4MiB", "k_alltoall_sessions", "AlltoAll+sessions R=8 B=4MiB"
    elif copy_engine:  # the same exchange by the copy engines (SDMA), no compute units for the bytes
        f = lambda: vr.vr_alltoall(comm, sw, 0, rw, 0, B, sig=0, flags=vr.VR_COLL_COPY_ENGINE,  # noqa: E731
                                   stream=stream)
        name, kernel, label = "alltoall_copy_engine_r8_4MiB", "sdma", "AlltoAll copy engine R=8 B=4MiB"
    else:
        f = lambda: vr.vr_alltoall(comm, sw, 0, rw, 0, B, sig=0, stream=stream)  # noqa: E731
        name, kernel, label = "alltoall_r8_4MiB", "k_alltoall", "AlltoAll R=8 B=4MiB"
    b.warm(f)
    rows[name] = row_entry(label, 2 * R * R * B, b.timed(f, reps, True), kernel, name)
    vr.vr_window_deregister(comm, sw)
    vr.vr_window_deregister(comm, rw)
    vr.vr_comm_destroy(comm)
    del s1, r1



def run_dispatch_row(b, reps, rows):
    import workloads as W
    vr, stream, torch = b.vr, b.stream.cuda_stream, b.torch
    c = W.CONFIGS["dispatch_r8_t4096_e256_k8"]
    R, T, H, E, K = c["ranks"], c["tokens"], c["hidden"], c["experts"], c["topk"]
    topk, x = W.dispatch_inputs(R, T, H, E, K, c["zipf_s"], seed=c["seed"])
    rb = H * 2
    cap = R * T * min(K, E // R)
    comm = comm_for(vr, R, signal_count=4)
    s1, xv = b.slices(R, T * rb, arrays=[x[r] for r in range(R)])
    r1, rv = b.slices(R, cap * rb, fill=0)
    xw = vr.vr_window_register(comm, [v.data_ptr() for v in xv], T * rb)
    rw = vr.vr_window_register(comm, [v.data_ptr() for v in rv], cap * rb)
    tk = torch.from_numpy(topk).cuda()
    counts = torch.zeros(R, E // R, dtype=torch.int32, device="cuda")
    src = torch.zeros(R, cap, dtype=torch.int32, device="cuda")
    f = lambda: vr.vr_dispatch(comm, xw, 0, rb, tk, T, K, E, rw, 0, cap, counts, src, None, 0, 1, stream=stream)  # noqa
    b.warm(f)
    nrows = int((topk >= 0).sum())
    bytes_alg = R * T * rb + topk.nbytes + nrows * rb + nrows * 4 + R * (E // R) * 4
    rows["dispatch_r8_t4096_e256_k8"] = row_entry("dispatch R=8 T=4096 512B E=256 K=8", bytes_alg,
                                                  b.timed(f, reps, True), "k_dispatch",
                                                  "dispatch_r8_t4096_e256_k8", {"rows": nrows})
    vr.vr_window_deregister(comm, xw)
    vr.vr_window_deregister(comm, rw)
    vr.vr_comm_destroy(comm)
    del s1, r1, tk, counts, src



def run_combine_row(b, reps, rows):
    import workloads as W
    vr, stream, torch = b.vr, b.stream.cuda_stream, b.torch
    c = W.CONFIGS["dispatch_r8_t4096_e256_k8"]
    R, T, H, E, K = c["ranks"], c["tokens"], c["hidden"], c["experts"], c["topk"]
    topk, x = W.dispatch_inputs(R, T, H, E, K, c["zipf_s"], seed=c["seed"])
    weights = W.router_weights(topk, E, c["zipf_s"])
    rb = H * 2
    cap = R * T * min(K, E // R)
    comm = comm_for(vr, R, signal_count=4)
    s1, xv = b.slices(R, T * rb, arrays=[x[r] for r in range(R)])
    r1, rv = b.slices(R, cap * rb, fill=0)
    o1, ov = b.slices(R, T * rb, fill=0)
    xw = vr.vr_window_register(comm, [v.data_ptr() for v in xv], T * rb)
    yw = vr.vr_window_register(comm, [v.data_ptr() for v in rv], cap * rb)
    ow = vr.vr_window_register(comm, [v.data_ptr() for v in ov], T * rb)
    tk = torch.from_numpy(topk).cuda()
    wt = torch.from_numpy(weights).cuda()
    counts = torch.zeros(R, E // R, dtype=torch.int32, device="cuda")
    src = torch.zeros(R, cap, dtype=torch.int32, device="cuda")
    pos = torch.zeros(R, T, K, dtype=torch.int32, device="cuda")
    # the dispatched token rows stand in for the expert outputs
    vr.vr_dispatch(comm, xw, 0, rb, tk, T, K, E, yw, 0, cap, counts, src, pos, 0, 1, stream=stream)
    f = lambda: vr.vr_combine(comm, yw, 0, cap, rb, vr.VR_DT_BF16, tk, wt, pos, T, K, E, ow, 0, 2,  # noqa: E731
                              stream=stream)
    b.warm(f)
    nrows = int((topk >= 0).sum())
    bytes_alg = nrows * rb + R * T * rb + 3 * topk.nbytes
    rows["combine_r8_t4096_e256_k8"] = row_entry("combine R=8 T=4096 512B E=256 K=8", bytes_alg,
                                                 b.timed(f, reps, True), "k_combine",
                                                 "combine_r8_t4096_e256_k8", {"rows": nrows})
    code, bits = vr.vr_comm_get_async_error(comm)
    if code != vr.VR_OK:
        raise RuntimeError(f"device error in the combine: {vr.vr_error_string(code)} bits={bits:#x}")
    for w in (xw, yw, ow):
        vr.vr_window_deregister(comm, w)
    vr.vr_comm_destroy(comm)
    del s1, r1, o1, tk, wt, counts, src, pos


def run_dedup_rows(b, reps, rows):
    """The per-rank (dedup) dispatch and its combine on the dispatch workload."""
    import workloads as W
    vr, stream, torch = b.vr, b.stream.cuda_stream, b.torch
    c = W.CONFIGS["dispatch_r8_t4096_e256_k8"]
    R, T, H, E, K = c["ranks"], c["tokens"], c["hidden"], c["experts"], c["topk"]
    topk, x = W.dispatch_inputs(R, T, H, E, K, c["zipf_s"], seed=c["seed"])
    rb = H * 2
    cap = R * T
    comm = comm_for(vr, R, signal_count=4)
    s1, xv = b.slices(R, T * rb, arrays=[x[r] for r in range(R)])
    r1, rv = b.slices(R, cap * rb, fill=0)
    o1, ov = b.slices(R, T * rb, fill=0)
    xw = vr.vr_window_register(comm, [v.data_ptr() for v in xv], T * rb)
    rw = vr.vr_window_register(comm, [v.data_ptr() for v in rv], cap * rb)
    ow = vr.vr_window_register(comm, [v.data_ptr() for v in ov], T * rb)
    tk = torch.from_numpy(topk).cuda()
    counts = torch.zeros(R, E // R, dtype=torch.int32, device="cuda")
    src = torch.zeros(R, cap, dtype=torch.int32, device="cuda")
    experts = torch.zeros(R, cap, K, dtype=torch.int32, device="cuda")
    pos = torch.zeros(R, T, R, dtype=torch.int32, device="cuda")
    fd = lambda: vr.vr_dispatch_dedup(comm, xw, 0, rb, tk, T, K, E, rw, 0, cap, counts, src, experts,  # noqa: E731
                                      pos, 0, 1, stream=stream)
    b.warm(fd)
    epr = E // R
    nrows = int(sum(len({int(e) // epr for e in topk[s, t] if e >= 0}) for s in range(R) for t in range(T)))
    bytes_d = R * T * rb + topk.nbytes + nrows * (rb + 4 + 4 * K) + R * epr * 4 + pos.numel() * 4
    rows["dispatch_dedup_r8_t4096_e256_k8"] = row_entry("dedup dispatch R=8 T=4096 512B E=256 K=8", bytes_d,
                                                        b.timed(fd, reps, True), "k_dispatch_dedup",
                                                        "dispatch_dedup_r8_t4096_e256_k8", {"rows": nrows})
    # combine: the dispatched rows stand in for each rank's mixed expert outputs
    fc = lambda: vr.vr_combine_dedup(comm, rw, 0, cap, rb, vr.VR_DT_BF16, pos, T, ow, 0, 2,  # noqa: E731
                                     stream=stream)
    fc()
    bytes_c = nrows * rb + R * T * rb + pos.numel() * 4
    rows["combine_dedup_r8_t4096_e256_k8"] = row_entry("dedup combine R=8 T=4096 512B E=256 K=8", bytes_c,
                                                       b.timed(fc, reps, True), "k_combine_dedup",
                                                       "combine_dedup_r8_t4096_e256_k8", {"rows": nrows})
    code, bits = vr.vr_comm_get_async_error(comm)
    if code != vr.VR_OK:
        raise RuntimeError(f"device error in the dedup rows: {vr.vr_error_string(code)} bits={bits:#x}")
    for w in (xw, rw, ow):
        vr.vr_window_deregister(comm, w)
    vr.vr_comm_destroy(comm)
    del s1, r1, o1, tk, counts, src, experts, pos


def run_allgather_row(b, reps, rows, copy_engine=False):
    import workloads as W
    vr, stream = b.vr, b.stream.cuda_stream
    c = W.CONFIGS["allgather_r16_64MiB"]
    R, M = c["ranks"], c["bytes_per_rank"]
    sends = W.allgather_inputs(R, M, seed=c["seed"])
    comm = comm_for(vr, R, signal_count=2)
    s1, sv = b.slices(R, M, arrays=sends)
    r1, rv = b.slices(R, R * M, fill=None)
    sw = vr.vr_window_register(comm, [v.data_ptr() for v in sv], M)
    rw = vr.vr_window_register(comm, [v.data_ptr() for v in rv], R * M)
    if copy_engine:  # the bytes moved by the copy engines (SDMA)
        f = lambda: vr.vr_allgather(comm, sw, 0, rw, 0, M, sig=0, flags=vr.VR_COLL_COPY_ENGINE,  # noqa: E731
                                    stream=stream)
        name, kernel, label, n = "allgather_copy_engine_r16_64MiB", "sdma", "AllGather copy engine R=16 M=64MiB", 2
    else:
        f = lambda: vr.vr_allgather(comm, sw, 0, rw, 0, M, sig=0, stream=stream)  # noqa: E731
        name, kernel, label, n = "allgather_r16_64MiB", "k_allgather", "AllGather R=16 M=64MiB", max(3, reps // 2)
    b.warm(f)
    rows[name] = row_entry(label, R * M + R * R * M, b.timed(f, n, True), kernel, name)
    vr.vr_window_deregister(comm, sw)
    vr.vr_window_deregister(comm, rw)
    vr.vr_comm_destroy(comm)
    del s1, r1



def run_put_get_rows(b, reps, rows):
    """One-sided put and get of 1 GiB between two ranks (a multi-workgroup coop):
    put with a SignalInc and a CounterInc, get with a CounterInc."""
    vr, stream = b.vr, b.stream.cuda_stream
    R, n = 2, 1 << 30
    comm = comm_for(vr, R, signal_count=2, counter_count=2)
    s1, sv = b.slices(R, n, fill=7)
    r1, rv = b.slices(R, n, fill=0)
    sw = vr.vr_window_register(comm, [v.data_ptr() for v in sv], n)
    rw = vr.vr_window_register(comm, [v.data_ptr() for v in rv], n)
    fp = lambda: vr.vr_put(comm, 0, 0, 1, rw, 0, sw, 0, n, vr.SignalInc(0), vr.CounterInc(0), stream=stream)  # noqa
    fg = lambda: vr.vr_get(comm, 0, 1, 0, sw, 0, rw, 0, n, vr.CounterInc(1), stream=stream)  # noqa: E731
    for name, label, f in (("put_1GiB", "put 1 GiB", fp), ("get_1GiB", "get 1 GiB", fg)):
        b.warm(f)
        rows[name] = row_entry(label, 2 * n, b.timed(f, max(3, reps // 2), True), "k_put", name)
    code, bits = vr.vr_comm_get_async_error(comm)
    if code != vr.VR_OK:
        raise RuntimeError(f"device error in put/get: {vr.vr_error_string(code)} bits={bits:#x}")
    vr.vr_window_deregister(comm, sw)
    vr.vr_window_deregister(comm, rw)
    vr.vr_comm_destroy(comm)
    del s1, r1


def run_pingpong_rows(b, reps, rows):
    """The control path of a small put: 2000 round trips of 256 B between two
    workgroups inside one kernel (put + SignalInc + wait each way), with the
    second rank on another XCD and on the same XCD, and between the two waves
    of one workgroup."""
    vr, stream = b.vr, b.stream.cuda_stream
    R, n, iters = 2, 256, 2000
    comm = comm_for(vr, R, signal_count=2)
    s1, sv = b.slices(R, 4096, fill=3)
    w = vr.vr_window_register(comm, [v.data_ptr() for v in sv], 4096)
    for name, label, flags in (("pingpong_cross_xcd_256B", "ping-pong 256 B, other XCD", 0),
                               ("pingpong_same_xcd_256B", "ping-pong 256 B, same XCD", vr.VR_PINGPONG_SAME_XCD),
                               ("pingpong_waves_256B", "ping-pong 256 B, two waves of one workgroup",
                                vr.VR_PINGPONG_WAVES)):
        f = lambda: vr.vr_signal_pingpong(comm, w, 0, n, iters, sig=0, flags=flags, stream=stream)  # noqa: E731
        b.warm(f)
        t = b.timed(f, max(3, reps // 2), False)
        med = float(np.median(t))
        rows[name] = row_entry(label, 4 * n * iters, t, "k_pingpong", name,
                               {"round_trips": iters, "us_per_round_trip": round(med * 1e3 / iters, 3)})
    code, bits = vr.vr_comm_get_async_error(comm)
    if code != vr.VR_OK:
        raise RuntimeError(f"device error in the ping-pong: {vr.vr_error_string(code)} bits={bits:#x}")
    vr.vr_window_deregister(comm, w)
    vr.vr_comm_destroy(comm)
    del s1


def run_ring_row(b, reps, rows, weak=False):
    import workloads as W
    vr, stream, torch = b.vr, b.stream.cuda_stream, b.torch
    c = W.CONFIGS["ring_r16_1Mi_x_256B"]
    R, P, pb, C = c["ranks"], c["puts_per_rank"], c["put_bytes"], c["contexts"]
    sends = W.ring_inputs(R, P, pb, seed=c["seed"])
    comm = comm_for(vr, R, signal_count=C, counter_count=C, context_count=C)
    s1, sv = b.slices(R, P * pb, arrays=sends)
    r1, rv = b.slices(R, P * pb, fill=0)
    sw = vr.vr_window_register(comm, [v.data_ptr() for v in sv], P * pb)
    rw = vr.vr_window_register(comm, [v.data_ptr() for v in rv], P * pb)
    lit = torch.zeros(2, dtype=torch.int64, device="cuda")
    flags = vr.VR_RING_WEAK if weak else 0
    f = lambda: vr.vr_ring_exchange(comm, sw, rw, pb, P, C, 0, 0, flags=flags, stream=stream)  # noqa: E731
    b.warm(f)
    t = b.timed(f, reps, True)
    med = float(np.median(t))
    # the litmus in a pass of its own, as the other rows' litmus runs in the
    # tests: one wavefront per (rank, context) checks each newly seen signal
    # value against the received bytes (its acquires and reads slow the
    # exchange, so it is timed apart)
    fl = lambda: vr.vr_ring_exchange(comm, sw, rw, pb, P, C, 0, 0, litmus=lit, flags=flags,  # noqa: E731
                                     stream=stream)
    b.warm(fl, 2)
    tl = b.timed(fl, max(3, reps // 2), True)
    lh = lit.cpu().numpy()
    # weak: litmus[1] counts observations the weak rule allows (a later message seen first)
    extra = {"Mputs_per_s": round(R * P / (med * 1e-3) / 1e6, 1), "litmus_checks": int(lh[0]),
             ("litmus_reorders_observed" if weak else "litmus_violations"): int(lh[1]),
             "with_litmus_median_ms": round(float(np.median(tl)), 5),
             "with_litmus_back_to_back_ms": round(tl.b2b_ms, 5)}
    name = "ring_weak_r16_1Mi_x_256B" if weak else "ring_r16_1Mi_x_256B"
    rows[name] = row_entry(f"ring{' (weak signals)' if weak else ''} R=16 2^20 puts x 256B", 2 * R * P * pb, t,
                           "k_ring_weak" if weak else "k_ring", name, extra)
    code, bits = vr.vr_comm_get_async_error(comm)
    if code != vr.VR_OK:
        raise RuntimeError(f"device error in the ring exchange: {vr.vr_error_string(code)} bits={bits:#x}")
    vr.vr_window_deregister(comm, sw)
    vr.vr_window_deregister(comm, rw)
    vr.vr_comm_destroy(comm)
    del s1, r1


def calib_copy(b: Bench, reps: int = 3):
    """A plain elementwise kernel of known traffic: reads 1 GiB, writes 1 GiB.

    Its FETCH_SIZE / WRITE_SIZE counters scale the same counters of our
    kernels to bytes (the kernel is torch's bitwise_not on int32)."""
    torch = b.torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        b.flush_cache()
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    log("calibration copy done (1 GiB read + 1 GiB write per launch)")


def copy_ceiling(b: Bench, reps: int = 5):
    """Context for the roofline: a plain device copy of 1 GiB (torch copy_),
    back to back, events on the stream; GB/s over the 2 GiB moved."""
    torch = b.torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    t = b.timed(lambda: dst.copy_(src), reps, False)
    med = float(np.median(t))
    del src, dst
    out = {"GBps": round(2 * n / (med * 1e-3) / 1e9, 1), "how": f"torch copy_ of 1 GiB on the device, median of {reps}"}
    out["library_put_1GiB_back_to_back_GBps"] = library_put_back_to_back(b)
    return out


def library_put_back_to_back(b: Bench, steps: int = 20):
    """The library's 1 GiB put (rank 0 -> 1, SignalInc) timed as the headline
    is: back to back between two events, no flush, so the dirty lines each
    call leaves in the Infinity Cache are written back inside the next. The
    flushed put rows run faster because their last writes still sit in that
    cache when the timer stops."""
    vr, stream = b.vr, b.stream.cuda_stream
    R, n = 2, 1 << 30
    comm = comm_for(vr, R, signal_count=1)
    s1, sv = b.slices(R, n, fill=7)
    r1, rv = b.slices(R, n, fill=0)
    sw = vr.vr_window_register(comm, [v.data_ptr() for v in sv], n)
    rw = vr.vr_window_register(comm, [v.data_ptr() for v in rv], n)

    def f():
        vr.vr_put(comm, 0, 0, 1, rw, 0, sw, 0, n, vr.SignalInc(0), stream=stream)

    b.warm(f)
    e0 = b.torch.cuda.Event(enable_timing=True)
    e1 = b.torch.cuda.Event(enable_timing=True)
    b.torch.cuda.synchronize()
    e0.record(b.stream)
    for _ in range(steps):
        f()
    e1.record(b.stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / steps
    code, bits = vr.vr_comm_get_async_error(comm)
    if code != vr.VR_OK:
        raise RuntimeError(f"device error in the put: {vr.vr_error_string(code)} bits={bits:#x}")
    vr.vr_window_deregister(comm, sw)
    vr.vr_window_deregister(comm, rw)
    vr.vr_comm_destroy(comm)
    del s1, r1
    gbs = 2 * n / (ms * 1e-3) / 1e9
    log(f"library put 1 GiB back to back: {gbs:.1f} GB/s ({ms:.4f} ms)")
    return round(gbs, 1)


# ---- the CPU oracle beside it ---------------------------------------------------------------------
def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(xs, R: int, N: int, budget_s: float = 30.0, target_s: float = 10.0):
    """Time the oracle's protocol simulation of the same AllReduce on one host core.

    Bounded sample: the first n elements of every rank's input, n growing
    until one run takes at least ~2 s (capped by the budget); runs of that
    sample are then repeated until about `target_s` seconds of timed CPU work
    (within the budget), and GB/s is the sample's algorithmic bytes over the
    mean of the repeats.
    """
    from oracle import primitives as P, protocol as pr
    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except (AttributeError, OSError):
        pass
    n = 1 << 20
    t_used = 0.0
    best = None
    while True:
        w = P.World(R, signal_count=1)
        sw = w.register([x[:n].view(np.uint8).copy() for x in xs])
        rw = w.register_zeros(n * 2)
        sc = w.register_zeros(pr.allreduce_scratch_bytes(n, R, "bf16"))
        t0 = time.perf_counter()
        pr.run(w, pr.allreduce_programs(w, sw, rw, sc, n, "bf16", 0), seed=0)
        dt = time.perf_counter() - t0
        t_used += dt
        best = (n, dt)
        del w
        if dt >= 2.0 or n >= N or t_used + 4 * dt > budget_s:
            break
        n = min(N, n * 4)
    n, dt = best
    # repeats of the chosen sample; the size-finding run is left out when
    # repeats fit the budget (a process's first runs pay one-time page faults)
    runs = []
    while sum(runs) < target_s and t_used + dt <= budget_s:
        w = P.World(R, signal_count=1)
        sw = w.register([x[:n].view(np.uint8).copy() for x in xs])
        rw = w.register_zeros(n * 2)
        sc = w.register_zeros(pr.allreduce_scratch_bytes(n, R, "bf16"))
        t0 = time.perf_counter()
        pr.run(w, pr.allreduce_programs(w, sw, rw, sc, n, "bf16", 0), seed=0)
        runs.append(time.perf_counter() - t0)
        t_used += runs[-1]
        del w
    if not runs:
        runs = [dt]
    dt = sum(runs) / len(runs)
    gbs = 2 * R * n * 2 / dt / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"protocol simulation of the bf16 AllReduce, R={R}, first {n} of {N} elements per rank, "
                      f"{len(runs)} runs, {sum(runs):.1f} s timed on one pinned host core (numpy single-threaded); "
                      f"value over the mean run ({dt:.2f} s)",
            "seconds": round(sum(runs), 3), "runs": len(runs), "host_cpu_count": os.cpu_count(),
            "host_cpu_model": cpu_model()}


def cpu_rows():
    """The oracle's plain definition of every other workload, timed on one host
    core on a bounded sample of its inputs (the sample is named; GB/s over the
    sample's algorithmic bytes; the best of a few runs for the short ones).
    Inputs are generated before the clock starts."""
    import workloads as W
    from oracle import definitions as D
    out = {}

    def clock(name, fn, nbytes, sample, runs=1):
        best = None
        for _ in range(runs):
            t0 = time.perf_counter()
            fn()
            dt = time.perf_counter() - t0
            best = dt if best is None else min(best, dt)
        out[name] = {"GBps": round(nbytes / best / 1e9, 3), "seconds": round(best, 4), "sample": sample}

    c = W.CONFIGS["allreduce_f32_r4_1Mi"]
    xs = W.allreduce_f32_inputs(c["ranks"], c["count"], run="B", seed=c["seed"])
    clock("allreduce_f32_r4_1Mi", lambda: D.allreduce(xs, "f32"), 2 * c["ranks"] * c["count"] * 4, "whole workload",
          runs=5)
    c = W.CONFIGS["alltoall_r8_4MiB"]
    R, B = c["ranks"], c["block_bytes"]
    sends = W.alltoall_inputs(R, B, seed=c["seed"])
    clock("alltoall_r8_4MiB", lambda: D.alltoall(sends, B), 2 * R * R * B, "whole workload", runs=3)
    del sends
    c = W.CONFIGS["dispatch_r8_t4096_e256_k8"]
    R, T, H, E, K = c["ranks"], c["tokens"], c["hidden"], c["experts"], c["topk"]
    topk, x = W.dispatch_inputs(R, T, H, E, K, c["zipf_s"], seed=c["seed"])
    n = int((topk >= 0).sum())
    clock("dispatch_r8_t4096_e256_k8", lambda: D.dispatch(topk, x, E),
          R * T * H * 2 + topk.nbytes + n * (H * 2 + 4), "whole workload")
    epr = E // R
    nd = int(sum(len({int(e) // epr for e in topk[s, t] if e >= 0}) for s in range(R) for t in range(T)))
    clock("dispatch_dedup_r8_t4096_e256_k8", lambda: D.dispatch_dedup(topk, x, E),
          R * T * H * 2 + topk.nbytes + nd * (H * 2 + 4 + 4 * K), "whole workload")
    Ts = 1024
    ts, xs_ = topk[:, :Ts].copy(), x[:, :Ts].copy()
    pos = D.dispatch_positions(ts, E)
    y = W.expert_outputs(D.dispatch_rows_per_rank(ts, E), H, seed=7)
    wts = W.router_weights(ts, E)
    ns = int((ts >= 0).sum())
    clock("combine_r8_t4096_e256_k8", lambda: D.combine(ts, wts, pos, y, E),
          ns * H * 2 + R * Ts * H * 2 + 3 * ts.nbytes, f"{Ts} of {T} tokens per rank")
    c = W.CONFIGS["allgather_r16_64MiB"]
    R, M = c["ranks"], c["bytes_per_rank"] // 4
    sends = W.allgather_inputs(R, M, seed=c["seed"])
    clock("allgather_r16_64MiB", lambda: D.allgather(sends), R * M + R * R * M, "16 MiB per rank (of 64 MiB)")
    del sends
    c = W.CONFIGS["ring_r16_1Mi_x_256B"]
    R, P, pb = c["ranks"], c["puts_per_rank"], c["put_bytes"]
    sends = W.ring_inputs(R, P, pb, seed=c["seed"])
    zero = [np.zeros(P * pb, np.uint8)] * R
    clock("ring_r16_1Mi_x_256B", lambda: D.ring(sends, zero, P, pb), 2 * R * P * pb, "whole workload", runs=3)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-rows", action="store_true", help="skip the other workloads")
    ap.add_argument("--rows", default=",".join(ROW_NAMES), help="comma-separated subset of " + ",".join(ROW_NAMES))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--reps", type=int, default=20, help="repetitions per other workload")
    ap.add_argument("--dispatch-phases", action="store_true",
                    help="print the dispatch's phase timeline (markdown) instead of the JSON line")
    ap.add_argument("--calib", action="store_true",
                    help="first run a plain 1 GiB read + 1 GiB write kernel (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the R virtual ranks share one device; runs across several GPUs "
              "are not supported", file=sys.stderr)
        sys.exit(2)
    b = Bench()
    if args.dispatch_phases:
        print(dispatch_phases(b, args.reps))
        print()
        print(dispatch_phases(b, args.reps, dedup=True))
        return
    if args.calib:
        calib_copy(b)
    head = run_allreduce_headline(b, args.steps, args.warmup)
    kern = float(np.mean(head["kern_ms"]))
    fl_med = float(np.median(head["flushed_ms"]))
    achieved = head["bytes_alg"] / (kern * 1e-3) / 1e9
    value = head["bytes_alg"] / (head["ms_per_step"] * 1e-3) / 1e9
    workload = "allreduce_bf16_r8_64Mi"
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(head["ms_per_step"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": workload, "ranks": head["R"], "count_per_rank": head["N"], "elem": "bf16",
                   "accumulate": "f32 in rank order", "algorithmic_bytes": head["bytes_alg"],
                   "frac_of_peak": round(value / HBM_PEAK_GBS, 4), "inputs": "seeded normal(0,1) -> bf16"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("k_allreduce", workload), "kernel": "k_allreduce",
                     "kernel_ms_mean": round(kern, 5),
                     # cold figure: median of 20 launches, each after a 1 GiB read flush (events
                     # around each launch, so the launch latency is included)
                     "kernel_ms_median_flushed": round(fl_med, 5), "reps_flushed": len(head["flushed_ms"]),
                     "frac_flushed": round(head["bytes_alg"] / (fl_med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if not args.no_rows:
        out["rows"] = run_rows(b, args.reps, tuple(args.rows.split(",")))
        out["copy_ceiling"] = copy_ceiling(b)
        if "put_1GiB" in out["rows"]:  # the library's own dwordx4 copy: a 1 GiB one-sided put
            out["copy_ceiling"]["library_put_1GiB_GBps"] = out["rows"]["put_1GiB"]["GBps"]
    if not args.no_cpu:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(head["xs"], head["R"], head["N"])
        if not args.no_rows:
            out["cpu_baseline"]["rows"] = cpu_rows()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
