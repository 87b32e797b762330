"""Benchmark of the weight-only low-bit matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only main]

A step is one qgemm call of the decode workload: INT4 asymmetric, group 128,
M=1, N=6144, K=2048 (the fused QKV of a D=2048 block).  Each step reads a
different copy of the packed weight, scales and zero points; the copies add
up to more than twice the 256 MB on-die cache, and a 512 MiB read evicts that
cache before every timed replay, so every timed step streams its weight bytes
from HBM whatever K is.  The K timed steps are captured once in a HIP graph
between two device clock stamps on the stream the kernels run on, and
replayed (median of several replays); four untimed steps on the last copies
open each graph, before the first stamp (the first kernel after the eviction
pays about 2 us on its own), and the span of an empty stamp pair (the first
stamp's own step) is taken off, so a step's time does not depend on K.
HIP events around the same replays are reported beside them.

One JSON line is printed: value = weight GB/s at M=1, plus the roofline of the
GEMV kernel against the published HBM peak and against the ceilings measured
in the same run (a plain streaming read of the same bytes, the empty-kernel
launch floor, the sustained MFMA rate), per-dispatch percentiles (from the
committed kernel-trace summary), the CPU
oracle timed on the host for every workload, and secondary legs (M=8, the
M=128 MFMA GEMM in TFLOP/s, INT2, q4_0, q8_0, q4k, the looped shared block).
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak, published
MALL_BYTES = 256 << 20         # on-die cache that rotating copies must exceed
SECONDARY_REPLAYS = 5          # secondary legs report the median of this many timed replays
MAIN_REPLAYS = 5               # the headline: median of this many timed replays
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
LOOP_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "loop_traffic.json")
DISPATCH_FILE = os.path.join(ROOT, "profiles", "dispatch.json")
_EVICT = {}


def evict(torch):
    """Read 512 MiB (twice the on-die cache) so that no weight bytes stay
    cached from earlier work; issued on the current stream, outside any graph.
    Reading, not writing: an eviction by writes leaves the cache full of dirty
    lines, whose write-back to HBM then competes with the timed reads that
    displace them (about 28 us per timed replay of 20 decode steps)."""
    buf = _EVICT.get("buf")
    if buf is None:
        buf = _EVICT["buf"] = torch.ones(2 * MALL_BYTES // 2, dtype=torch.float16, device="cuda")
        for _ in range(2):   # the writes above leave dirty lines: read them out once
            torch.sum(buf, dtype=torch.float32)
        torch.cuda.synchronize()
    torch.sum(buf, dtype=torch.float32)


KERNEL_SRC = os.path.join(ROOT, "bit_weight_only_dequant_amd", "csrc", "kernels.hip")


def kernel_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=810)
    ap.add_argument("--warmup", type=int, default=81)
    ap.add_argument("--only", choices=["all", "main", "gemm", "int2", "loop", "loop_prof", "loop_prof_persistent", "fp16",
                                       "copy", "stream", "floor"],
                    default="all",
                    help="main/gemm/int2/loop/fp16/stream/floor: run one leg (for profiler runs; int2: INT2 g64 at "
                         "M=1); copy: the calibration copy; loop_prof: the looped block resident and with the cache "
                         "evicted between loops")
    ap.add_argument("--loop-m", type=int, default=128, help="M of --only loop / loop_prof")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=5, help="oracle timings per workload and thread count")
    return ap.parse_args()


class Leg:
    """One workload with `copies` rotating weight copies resident on the GPU."""

    def __init__(self, qgm, torch, case, M, min_bytes=2 * MALL_BYTES, max_copies=256):
        self.torch, self.qgm = torch, qgm
        self.case, self.M = case, M
        base = qgm.QuantLinear.from_case(case, "cuda")
        self.wbytes = base.weight_bytes
        self.copies = max(1, min(max_copies, -(-min_bytes // self.wbytes))) if min_bytes else 1
        self.lins = [base]
        for _ in range(self.copies - 1):
            c = object.__new__(qgm.QuantLinear)
            c.__dict__.update(base.__dict__)
            c.packed = base.packed.clone()
            c.scales = base.scales.clone()
            c.zeros = None if base.zeros is None else base.zeros.clone()
            self.lins.append(c)
        self.x = qgm.to_half_tensor(case.x[:M], "cuda")
        self.y = torch.empty((M, case.N), dtype=torch.float16, device="cuda")

    def step(self, i):
        self.lins[i % self.copies](self.x, out=self.y)

    def time(self, steps, warmup, replays=1):
        """ms per step: the median over `replays` timed replays of a graph of
        `steps` calls, each replay preceded by an eviction of the on-die cache
        (outside the timed region), so no step finds its weights cached
        whatever `steps` is."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        g, stamps = capture(self.qgm, torch, self.step, steps)
        self.replay_ms, self.replay_ms_events = replay_times(torch, g, steps, replays, stamps)
        return float(np.median(self.replay_ms))


class Stamps:
    """Two device clock stamps (qg_clock_stamp) around the steps of a graph."""

    def __init__(self, qgm, torch):
        self.qgm = qgm
        self.buf = torch.zeros(2, dtype=torch.int64, device="cuda")
        self.khz = qgm.clock_rate_khz(torch.cuda.current_device())

    def first(self):
        self.qgm.clock_stamp(self.buf[0:1])

    def last(self):
        self.qgm.clock_stamp(self.buf[1:2])

    def span_ms(self):
        t = self.buf.cpu().tolist()
        return (t[1] - t[0]) / self.khz


WARM_STEPS = 4   # untimed steps inside each graph, before its first stamp


def capture(qgm, torch, step, steps, warm=WARM_STEPS):
    """`steps` calls of step(i) captured in one HIP graph between two device
    clock stamps; the first replay (which uploads the graph) is not timed.
    Before the first stamp the graph runs `warm` untimed calls step(-1),
    step(-2), ...: the steps rotate over copies (i % copies), so these read
    the last copies, far from the first timed ones, and the timed steps still
    find their weights evicted.  They take up what the first kernels after
    the eviction pay on their own: about 2 us more than a running call
    (decode GEMV: 6.0 against 3.84 us at one step), whichever kernels they are
    (after four empty kernels the one timed GEMV takes 4.4 us, after another
    GEMV 4.0-4.1 us), which would otherwise make a step's time depend on K."""
    stamps = Stamps(qgm, torch)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for j in range(warm):
            step(-1 - j)
        stamps.first()
        for i in range(steps):
            step(i)
        stamps.last()
    g.replay()
    torch.cuda.synchronize()
    return g, stamps


_STAMP_PAIR = {}


def stamp_pair_ms(qgm, torch, replays=9):
    """Span of the two clock stamps with nothing between them, under the same
    protocol (median of `replays` replays, each after an eviction): the first
    stamp's own step (its kernel and the launch gap after it), which every
    stamp span holds once on top of its K steps.  Measured once per process."""
    if "ms" not in _STAMP_PAIR:
        g, stamps = capture(qgm, torch, lambda i: None, 0, warm=0)
        spans = []
        for _ in range(replays):
            evict(torch)
            g.replay()
            torch.cuda.synchronize()
            spans.append(stamps.span_ms())
        _STAMP_PAIR["ms"] = float(np.median(spans))
    return _STAMP_PAIR["ms"]


def replay_times(torch, g, steps, replays, stamps):
    """ms per step of each of `replays` timed replays of graph g, the on-die
    cache evicted before each: from the device clock stamps inside the graph
    (the stamp span less the span of an empty stamp pair, so exactly the K
    steps), and from HIP events recorded on the stream around the replay (the
    steps plus the first stamp and the graph's own launch latency, about 11 us
    per replay on this runtime, which only an event recorded inside the graph
    could exclude, and the runtime refuses event records during capture)."""
    pair = stamp_pair_ms(stamps.qgm, torch)
    stream = torch.cuda.current_stream()
    inner, events = [], []
    for _ in range(replays):
        evict(torch)
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        g.replay()
        stop.record(stream)
        stop.synchronize()
        events.append(start.elapsed_time(stop) / steps)
        inner.append((stamps.span_ms() - pair) / steps)
    return inner, events


FORMAT_NAMES = ("int4_asym", "int2_asym", "q4_0", "q8_0", "q4k")


def leg_result(name, leg, ms, M, replays=1):
    c = leg.case
    flops = 2.0 * M * c.N * c.K
    r = dict(leg=name, M=M, N=c.N, K=c.K, format=FORMAT_NAMES[c.fmt],
             group=c.group, us_per_call=round(ms * 1e3, 3),
             weight_GBps=round(leg.wbytes / (ms * 1e-3) / 1e9, 1),
             TFLOPs=round(flops / (ms * 1e-3) / 1e12, 2), weight_copies=leg.copies)
    if replays > 1:
        r["timed_replays"] = replays   # us_per_call is their median
    r["hbm_frac"] = round(r["weight_GBps"] / HBM_PEAK_GBS, 4)
    r["mfma_frac"] = round(r["TFLOPs"] / MFMA_F16_PEAK_TFLOPS, 4)
    return r


CPU_WORKLOADS = (("tiny_int4_g32", 1), ("tiny_int4_g32", 4), ("decode_int4_g128", 1), ("decode_int4_g128", 8),
                 ("prefill_int4_g128", 128), ("int2_g64", 1), ("int2_g64", 128), ("q4_0_b32", 1),
                 ("q4_0_b32", 128))


def cpu_baseline(synth, reps):
    """The oracle as it stands, timed on the host for every workload: one
    oracle call per sample (one loop of the block for the looped workload),
    `reps` samples with every BLAS thread and `reps` with one, the median of
    each.  The headline is the decode workload at M = 1 on every thread."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])

    def timed(fn, min_s=0.2):
        calls, t0 = 0, time.perf_counter()
        while True:
            fn()
            calls += 1
            el = time.perf_counter() - t0
            if el >= min_s or calls >= 1 and el >= 0.05 and calls * 50 > 1e4:
                return el / calls

    rows = []
    for name, M in CPU_WORKLOADS:
        c = synth.workload(name)
        x = c.x[:M]
        fn = lambda c=c, x=x, M=M: oracle.qgemm_ref(x, c.words, c.scales, c.zeros, M, c.N, c.K, c.group, c.fmt)
        r = dict(workload=name, M=M, N=c.N, K=c.K, weight_bytes=c.weight_bytes)
        for tag, lim in (("all", None), ("1", 1)):
            with threadpool_limits(limits=lim):
                sec = float(np.median([timed(fn) for _ in range(reps)]))
            r[f"s_per_call_{tag}"] = round(sec, 5)
            r[f"GBps_{tag}"] = round(c.weight_bytes / sec / 1e9, 4)
            r[f"TFLOPs_{tag}"] = round(2.0 * M * c.N * c.K / sec / 1e12, 6)
        rows.append(r)
    # the looped block: one loop (four linears and two residual adds) per sample
    lc = synth.loop_workload(M=128, L=1)
    lin = [dict(words=q.words, scales=q.scales, zeros=q.zeros, N=q.N, K=q.K, group=q.group, fmt=q.fmt)
           for q in lc.linears()]
    D = lc.x0.shape[1]
    wb = sum(q.weight_bytes for q in lc.linears())
    r = dict(workload="loop_block_int4_g128", M=128, D=D, L_sampled=1, weight_bytes_per_loop=wb)
    for tag, lim in (("all", None), ("1", 1)):
        with threadpool_limits(limits=lim):
            sec = float(np.median([timed(lambda: oracle.loop_block_ref(lc.x0, lin, 1, D=D), 0.0)
                                   for _ in range(reps)]))
        r[f"s_per_loop_{tag}"] = round(sec, 4)
        r[f"GBps_{tag}"] = round(wb / sec / 1e9, 4)
    rows.append(r)
    head = next(r for r in rows if r["workload"] == "decode_int4_g128" and r["M"] == 1)
    return dict(value=head["GBps_all"], unit="GB/s", cores=int(blas_threads), host_cpus=os.cpu_count(),
                kind="oracle", value_1thread=head["GBps_1"],
                sample=f"median of {reps} timings per workload and thread count; each timing is one oracle call "
                       f"(repeated to >= 0.2 s for the tiny workload; unpack, fp32 dequant, fp64 product) on the "
                       f"full workload, one loop of L for the looped block; 'all' = BLAS pool of {blas_threads} "
                       f"threads (the unpack and dequant are single-threaded numpy), '1' = one BLAS thread; "
                       f"headline: decode M=1 N=6144 K=2048 INT4 g128 on all threads",
                workloads=rows)


def loop_leg(qgm, torch, synth, L=8, M=128, control=True):
    """Looped shared block: per-loop time with the on-die cache evicted once
    before loop 1 ("cold": loops 2..L find the shared weights where loop 1 left
    them), with it warm, and -- the control -- with the cache evicted before
    every loop (outside the timed loops), so every loop streams its weights
    from HBM.  M = 128 is the prefill-sized block; M = 1 the decode step."""
    lc = synth.loop_workload(M=M, L=L)
    lins = [qgm.QuantLinear.from_case(c, "cuda") for c in lc.linears()]
    x0 = qgm.to_half_tensor(lc.x0, "cuda")
    M, D = lc.x0.shape
    F = lc.up.N
    scratch = torch.empty(M * (3 * D + D + F), dtype=torch.float16, device="cuda")
    x = x0.clone()
    qgm.loop_block(x, lins, L, scratch=scratch)  # warm-up, allocates the workspace
    torch.cuda.synchronize()
    res = {}
    for mode in ("cold", "warm"):
        x.copy_(x0)
        if mode == "cold":
            evict(torch)
        else:
            qgm.loop_block(x, lins, 1, scratch=scratch)
            x.copy_(x0)
        events = [torch.cuda.Event(enable_timing=True) for _ in range(L + 1)]
        qgm.loop_block(x, lins, L, scratch=scratch, events=events)
        events[-1].synchronize()
        res[mode] = [events[i].elapsed_time(events[i + 1]) for i in range(L)]
    if control:
        x.copy_(x0)
        per = []
        for _ in range(L):
            evict(torch)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            qgm.loop_block(x, lins, 1, scratch=scratch, events=ev)
            ev[-1].synchronize()
            per.append(ev[0].elapsed_time(ev[1]))
        res["evict"] = per
    if M == 1:   # the same loops as one launch each, grid barriers between the four GEMVs
        status = torch.zeros(4, dtype=torch.int32, device="cuda")
        qgm.loop_block_persistent(x, lins, 1, scratch=scratch, status=status)   # warm-up
        for mode in ("cold", "evict"):
            x.copy_(x0)
            per = []
            if mode == "cold":
                evict(torch)
                events = [torch.cuda.Event(enable_timing=True) for _ in range(L + 1)]
                qgm.loop_block_persistent(x, lins, L, scratch=scratch, status=status, events=events)
                events[-1].synchronize()
                per = [events[i].elapsed_time(events[i + 1]) for i in range(L)]
            else:
                for _ in range(L):
                    evict(torch)
                    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                    qgm.loop_block_persistent(x, lins, 1, scratch=scratch, status=status, events=ev)
                    ev[-1].synchronize()
                    per.append(ev[0].elapsed_time(ev[1]))
            if int(status[0]) != 0:
                raise RuntimeError("qloop_block_persistent: a grid barrier gave up")
            res["persistent_" + mode] = per
        # both persistent forms timed in graphs too, as the four-launch block is below
        status.zero_()
        for key, one in (("graph_persistent", False), ("graph_persistent_one_launch", True)):
            def run_p(xx, ll, n, sc, one=one):
                qgm.loop_block_persistent(xx, ll, n, scratch=sc, status=status, one_launch=one)
            res[key] = loop_graph_times(qgm, torch, x, x0, lins, L, scratch, run=run_p)
        torch.cuda.synchronize()
        if int(status[0]) != 0:
            raise RuntimeError("qloop_block_persistent (graph): a grid barrier gave up")
        # all L loops in one launch (each XCD keeps its rows' weights in its L2)
        x.copy_(x0)
        evict(torch)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        qgm.loop_block_persistent(x, lins, L, scratch=scratch, status=status, events=ev[:1] + [None] * (L - 1) + ev[1:],
                                  one_launch=True)
        ev[-1].synchronize()
        if int(status[0]) != 0:
            raise RuntimeError("qloop_block_persistent (one launch): a grid barrier gave up")
        res["persistent_one_launch_total"] = ev[0].elapsed_time(ev[1])
    graph = loop_graph_times(qgm, torch, x, x0, lins, L, scratch)
    wbytes = sum(l.weight_bytes for l in lins)
    flops = 2.0 * M * (D * 3 * D + D * D + D * F + F * D)
    cold, warm = res["cold"], res["warm"]
    name = "loop_block_int4_g128" + ("" if M == 128 else f"_M{M}")
    out = dict(leg=name, M=M, D=D, F=F, L=L,
               weight_bytes_per_loop=wbytes,
               cold_loop_ms=[round(v, 4) for v in cold], warm_loop_ms=[round(v, 4) for v in warm],
               loop1_cold_ms=round(cold[0], 4),
               loops2_L_ms=round(float(np.median(cold[1:])), 4),   # median: robust to launch jitter
               TFLOPs_loops2_L=round(flops / (float(np.median(cold[1:])) * 1e-3) / 1e12, 2),
               weight_GBps_loop1_cold=round(wbytes / (cold[0] * 1e-3) / 1e9, 1))
    if control:
        ev_ms = float(np.median(res["evict"]))
        out.update(evict_each_loop_ms=[round(v, 4) for v in res["evict"]],
                   evict_each_loop_median_ms=round(ev_ms, 4),
                   weight_GBps_evict_each_loop=round(wbytes / (ev_ms * 1e-3) / 1e9, 1))
    if "persistent_cold" in res:
        pc, pe = res["persistent_cold"], res["persistent_evict"]
        out.update(persistent_cold_loop_ms=[round(v, 4) for v in pc],
                   persistent_loop1_cold_ms=round(pc[0], 4),
                   persistent_loops2_L_ms=round(float(np.median(pc[1:])), 4),
                   persistent_evict_each_loop_median_ms=round(float(np.median(pe)), 4))
        out["persistent_one_launch_ms_per_loop"] = round(res["persistent_one_launch_total"] / L, 4)
        out["graph_persistent"] = res["graph_persistent"]
        out["graph_persistent_one_launch"] = res["graph_persistent_one_launch"]
    out["graph"] = dict(graph, weight_GBps_loop1_cold=round(wbytes / (graph["loop1_cold_us"] * 1e-6) / 1e9, 1))
    if graph["loops2_L_us"]:
        out["graph"]["TFLOPs_loops2_L"] = round(flops / (graph["loops2_L_us"] * 1e-6) / 1e12, 2)
    hb = load_loop_traffic(name)
    if hb is not None:
        out["residency_counters"] = hb   # L2 fetch bytes and latency per loop (profiles/loop_traffic.json)
    return out


def loop_graph_times(qgm, torch, x, x0, lins, L, scratch, replays=5, run=None):
    """Per-loop GPU time of the looped block with no host launch cost in it:
    L loops, one loop and no loop each captured in a HIP graph between two
    device clock stamps (after one untimed loop on a copy of the weights),
    every replay after x is reset and the on-die cache evicted (outside the
    graph).  Loop 1 (cold: weights from HBM, the same as
    a loop after an eviction) = T_1 - T_0; loops 2..L (weights where loop 1
    left them) = (T_L - T_1) / (L - 1); medians over the replays.  The eager
    per-loop events above also time the host's launches, which at M = 1 take
    about as long as the four GEMVs.  run(x, linears, loops, scratch) runs the
    block (default: loop_block, four launches per loop)."""
    if run is None:
        def run(xx, ll, n, sc):
            qgm.loop_block(xx, ll, n, scratch=sc)
    # one untimed loop on a copy of the block's weights opens every graph, so
    # the first timed kernel does not pay what the first kernels after the
    # eviction pay (see capture); the block's own weights stay evicted
    warm_lins = []
    for l in lins:
        w = object.__new__(type(l))
        w.__dict__.update(l.__dict__)
        w.packed = l.packed.clone()
        w.scales = l.scales.clone()
        w.zeros = None if l.zeros is None else l.zeros.clone()
        warm_lins.append(w)
    warm_x = x0.clone()
    warm_scratch = torch.empty_like(scratch)

    def cap(nloops):
        stamps = Stamps(qgm, torch)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(warm_x, warm_lins, 1, warm_scratch)
            stamps.first()
            if nloops:
                run(x, lins, nloops, scratch)
            stamps.last()
        x.copy_(x0)
        g.replay()
        torch.cuda.synchronize()
        return g, stamps
    graphs = {n: cap(n) for n in sorted({0, 1, L})}
    t = {n: [] for n in graphs}
    for _ in range(replays):
        for n, (g, st) in graphs.items():
            x.copy_(x0)
            warm_x.copy_(x0)
            evict(torch)
            g.replay()
            torch.cuda.synchronize()
            t[n].append(st.span_ms() * 1e3)
    t0, t1, tl = (np.asarray(t[n]) for n in (0, 1, L))
    out = dict(loop1_cold_us=round(float(np.median(t1 - t0)), 3), stamp_pair_us=round(float(np.median(t0)), 3),
               replays=replays)
    out["loops2_L_us"] = round(float(np.median((tl - t1) / (L - 1))), 3) if L > 1 else None
    return out


def loop_prof(qgm, torch, synth, L=8, M=128):
    """For the HBM byte counters: the looped block once resident (cache
    evicted before loop 1 only), then L single loops each after an eviction.
    The evictions are fill kernels between the qGEMM dispatches."""
    lc = synth.loop_workload(M=M, L=L)
    lins = [qgm.QuantLinear.from_case(c, "cuda") for c in lc.linears()]
    x0 = qgm.to_half_tensor(lc.x0, "cuda")
    D, F = lc.x0.shape[1], lc.up.N
    scratch = torch.empty(M * (3 * D + D + F), dtype=torch.float16, device="cuda")
    x = x0.clone()
    qgm.loop_block(x, lins, 1, scratch=scratch)  # allocates the workspace
    x.copy_(x0)
    evict(torch)
    qgm.loop_block(x, lins, L, scratch=scratch)
    x.copy_(x0)
    for _ in range(L):
        evict(torch)
        qgm.loop_block(x, lins, 1, scratch=scratch)
    torch.cuda.synchronize()
    print(json.dumps(dict(loop_prof=True, M=M, L=L)), flush=True)


def loop_prof_persistent(qgm, torch, synth, L=8, reps=3):
    """For the counters: the M = 1 block in one persistent launch, `reps`
    times for one loop and `reps` times for L loops, each after an eviction."""
    lc = synth.loop_workload(M=1, L=L)
    lins = [qgm.QuantLinear.from_case(c, "cuda") for c in lc.linears()]
    x0 = qgm.to_half_tensor(lc.x0, "cuda")
    D, F = lc.x0.shape[1], lc.up.N
    scratch = torch.empty(3 * D + D + F, dtype=torch.float16, device="cuda")
    status = torch.zeros(4, dtype=torch.int32, device="cuda")
    x = x0.clone()
    for loops in [1] * reps + [L] * reps:
        x.copy_(x0)
        evict(torch)
        qgm.loop_block_persistent(x, lins, loops, scratch=scratch, status=status, one_launch=True)
    torch.cuda.synchronize()
    assert int(status[0]) == 0
    print(json.dumps(dict(loop_prof_persistent=True, L=L, reps=reps)), flush=True)


def stream_leg(qgm, torch, nbytes, steps, replays, grids=(256, 512, 1024, 2048)):
    """The streaming-read ceiling of one launch over `nbytes` (the headline's
    weight bytes): rotating slices of a buffer larger than twice the on-die
    cache, the same graph and eviction protocol as the qGEMM legs; the best
    grid of `grids` is the ceiling."""
    stride = -(-nbytes // 256) * 256
    copies = max(1, -(-2 * MALL_BYTES // stride))
    buf = torch.empty(copies * stride, dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    sink = torch.zeros(max(grids), dtype=torch.int32, device="cuda")
    best = None
    rows = []
    for wg in grids:
        def step(i, wg=wg):
            qgm.stream_read(buf[(i % copies) * stride:], nbytes, sink, wg)
        for i in range(4):
            step(i)
        torch.cuda.synchronize()
        g, stamps = capture(qgm, torch, step, steps)
        inner, events = replay_times(torch, g, steps, replays, stamps)
        ms = float(np.median(inner))
        gbs = nbytes / (ms * 1e-3) / 1e9
        rows.append(dict(workgroups=wg, us_per_launch=round(ms * 1e3, 3), GBps=round(gbs, 1),
                         us_per_launch_events=round(float(np.median(events)) * 1e3, 3)))
        if best is None or gbs > best["GBps"]:
            best = rows[-1]
        del g
    return dict(bytes_per_launch=nbytes, copies=copies, best=best, grids=rows)


def empty_floor(qgm, torch, workgroups, threads, steps, replays):
    """us per launch of an empty kernel of the given grid, in a graph."""
    for _ in range(4):
        qgm.empty_launch(workgroups, threads)
    torch.cuda.synchronize()
    g, stamps = capture(qgm, torch, lambda i: qgm.empty_launch(workgroups, threads), steps)
    inner, events = replay_times(torch, g, steps, replays, stamps)
    return dict(workgroups=workgroups, threads=threads, us_per_launch=round(float(np.median(inner)) * 1e3, 3),
                us_per_launch_events=round(float(np.median(events)) * 1e3, 3))


def mfma_peaks(qgm, torch):
    """The dense fp16 MFMA peak from the device's compute units and clock (4
    SIMDs per CU, 16*16*32*2 flops per 16-cycle v_mfma_f32_16x16x32_f16 per
    SIMD = 4096 flops per CU per cycle), and the rate the probe sustains."""
    info = qgm.device_info(0)
    derived = info["compute_units"] * 4096 * info["clock_khz"] * 1e3 / 1e12
    wg = info["compute_units"] * 2          # 8 waves per CU: 2 per SIMD
    iters = 4000
    out = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
    qgm.mfma_probe(out, wg, 10)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        qgm.mfma_probe(out, wg, iters)
        b.record(stream)
        b.synchronize()
        times.append(a.elapsed_time(b))
    ms = float(np.median(times))
    flops = wg * 4 * iters * qgm.MFMA_PROBE_FLOPS
    return dict(device=info, derived_TFLOPs=round(derived, 1),
                sustained_TFLOPs=round(flops / (ms * 1e-3) / 1e12, 1), published_TFLOPs=MFMA_F16_PEAK_TFLOPS,
                probe=f"{wg} workgroups x 4 waves x {iters} rounds of 16 independent v_mfma_f32_16x16x32_f16")


def graph_time(qgm, torch, step, steps, warmup):
    """ms per step of `step(i)`, captured once in a HIP graph and replayed
    once after an eviction of the on-die cache."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    g, stamps = capture(qgm, torch, step, steps)
    return replay_times(torch, g, steps, 1, stamps)[0][0]


def fp16_leg(qgm, torch, synth, Ms=(1, 8, 32, 128, 512, 2048)):
    """The fused qGEMM against two FP16 alternatives on the up-projection shape
    (INT4 g128, N=8192, K=2048): dequantize-at-load (qg_dequant to an fp16 W,
    then torch's fp16 GEMM, every call) and an FP16 body whose fp16 weights stay
    resident (torch's fp16 GEMM alone).  Weights rotate over copies larger than
    the on-die cache in all three, so each call reads its weights from HBM."""
    c = synth.workload("prefill_int4_g128")
    N, K = c.N, c.K
    base = qgm.QuantLinear.from_case(c, "cuda")
    w16 = qgm.dequant(base.packed, base.scales, base.zeros, N, K, c.group, c.fmt)
    n16 = max(1, -(-2 * MALL_BYTES // (N * K * 2)))
    w16s = [w16.clone() for _ in range(n16)]
    wtmp = torch.empty_like(w16)
    rows = []
    for M in Ms:
        xs = synth.draw_x(np.random.default_rng(7 + M), M, K)
        x = qgm.to_half_tensor(xs, "cuda")
        leg = Leg(qgm, torch, c, M)
        leg.x = x
        leg.y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        steps = 200 if M <= 128 else 50
        t_fused = leg.time(steps, 10)
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")

        def deq_step(i, leg=leg, x=x, y=y):
            lin = leg.lins[i % leg.copies]
            qgm.dequant_into(lin.packed, lin.scales, lin.zeros, N, K, c.group, c.fmt, wtmp)
            torch.matmul(x, wtmp.t(), out=y)

        def f16_step(i, x=x, y=y):
            torch.matmul(x, w16s[i % n16].t(), out=y)

        t_deq = graph_time(qgm, torch, deq_step, steps, 10)
        t_f16 = graph_time(qgm, torch, f16_step, steps, 10)
        fl = 2.0 * M * N * K
        rows.append(dict(M=M, fused_us=round(t_fused * 1e3, 2), dequant_then_fp16_us=round(t_deq * 1e3, 2),
                         fp16_resident_us=round(t_f16 * 1e3, 2),
                         fused_TFLOPs=round(fl / (t_fused * 1e-3) / 1e12, 1),
                         fp16_resident_TFLOPs=round(fl / (t_f16 * 1e-3) / 1e12, 1)))
        del leg
        torch.cuda.empty_cache()
    return dict(leg="fp16_comparison_int4_g128_N8192_K2048", fp16_weight_copies=n16, rows=rows,
                note="fp16 GEMM = torch.matmul (hipBLASLt), untuned, as a comparison only")


def calibration_copy(torch, nbytes=512 << 20, reps=3):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    a = torch.ones(nbytes // 2, dtype=torch.float16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps(dict(calibration_copy_bytes=nbytes, reps=reps)), flush=True)


def load_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy), or None when the
    kernel sources changed since the counters were taken."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except Exception:
        return None
    if t.get("kernel_src_sha") != kernel_hash():
        return None  # counters were taken on other kernel code
    entry = t.get(kernel)
    return None if entry is None else entry.get("bytes")


def load_dispatch(kernel):
    """Per-dispatch duration percentiles (us) of `kernel` from the committed
    kernel-trace summary, or None when the kernel sources changed since."""
    try:
        t = json.load(open(DISPATCH_FILE))
    except Exception:
        return None
    if t.get("kernel_src_sha") != kernel_hash():
        return None
    return t.get(kernel)


def load_loop_traffic(leg):
    """Per-loop HBM bytes of the looped block from the committed counter
    summary (resident loops and the evict-every-loop control), or None when
    the kernel sources changed since the counters were taken."""
    try:
        t = json.load(open(LOOP_TRAFFIC_FILE))
    except Exception:
        return None
    if t.get("kernel_src_sha") != kernel_hash():
        return None
    return t.get(leg)


def gemv_kernel_name(qgm, c):
    """The M = 1 kernel the library's plan picks: 16-row or 8-row workgroups."""
    rows = qgm.plan(1, c.N, c.K, c.group, c.fmt)["tile_n"]
    return "gemv_half_kernel<INT4> (8-row workgroups)" if rows == 8 else "gemv_kernel<INT4,1>"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the qGEMM would shard along N across GPUs with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_weight_only_dequant_amd as qgm
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.only == "copy":
        calibration_copy(torch)
        return

    main_case = synth.workload("decode_int4_g128")
    if args.only == "gemm":
        c = synth.workload("prefill_int4_g128")
        leg = Leg(qgm, torch, c, 128)
        ms = leg.time(max(64, args.steps // 8), 8, replays=SECONDARY_REPLAYS)
        print(json.dumps(leg_result("prefill_int4_g128_M128", leg, ms, 128, SECONDARY_REPLAYS)), flush=True)
        return
    if args.only == "int2":
        c = synth.workload("int2_g64")
        leg = Leg(qgm, torch, c, 1)
        ms = leg.time(args.steps, args.warmup, replays=SECONDARY_REPLAYS)
        print(json.dumps(leg_result("int2_g64_M1", leg, ms, 1, SECONDARY_REPLAYS)), flush=True)
        return
    if args.only == "loop":
        print(json.dumps(loop_leg(qgm, torch, synth, M=args.loop_m)), flush=True)
        return
    if args.only == "loop_prof":
        loop_prof(qgm, torch, synth, M=args.loop_m)
        return
    if args.only == "loop_prof_persistent":
        loop_prof_persistent(qgm, torch, synth)
        return
    if args.only == "fp16":
        print(json.dumps(fp16_leg(qgm, torch, synth)), flush=True)
        return
    if args.only == "stream":
        print(json.dumps(stream_leg(qgm, torch, main_case.weight_bytes, args.steps, MAIN_REPLAYS)), flush=True)
        return
    if args.only == "floor":
        pl = qgm.plan(1, main_case.N, main_case.K, main_case.group, main_case.fmt)
        print(json.dumps(empty_floor(qgm, torch, pl["workgroups"], 512, args.steps, MAIN_REPLAYS)), flush=True)
        return

    leg = Leg(qgm, torch, main_case, 1)
    ms = leg.time(args.steps, args.warmup, replays=MAIN_REPLAYS)
    main_r = leg_result("decode_int4_g128_M1", leg, ms, 1)
    if args.only == "main":
        print(json.dumps(main_r), flush=True)
        return
    replay_ms = list(leg.replay_ms)
    ms_events = float(np.median(leg.replay_ms_events))
    wbytes, copies = leg.wbytes, leg.copies
    del leg
    torch.cuda.empty_cache()

    # ceilings measured in the same run
    stream = stream_leg(qgm, torch, wbytes, args.steps, MAIN_REPLAYS)
    pl = qgm.plan(1, main_case.N, main_case.K, main_case.group, main_case.fmt)
    floor = empty_floor(qgm, torch, pl["workgroups"], 512, args.steps, MAIN_REPLAYS)
    peaks = mfma_peaks(qgm, torch)
    torch.cuda.empty_cache()

    secondary = []
    leg8 = Leg(qgm, torch, main_case, 8)
    secondary.append(leg_result("decode_int4_g128_M8", leg8, leg8.time(400, 40, SECONDARY_REPLAYS), 8, SECONDARY_REPLAYS))
    del leg8
    for name, M in (("prefill_int4_g128", 128), ("int2_g64", 1), ("int2_g64", 128),
                    ("q4_0_b32", 1), ("q4_0_b32", 128), ("q8_0_b32", 1), ("q8_0_b32", 128),
                    ("q4k_s256", 1), ("q4k_s256", 128)):
        c = synth.workload(name)
        leg2 = Leg(qgm, torch, c, M)
        steps = 400 if M == 1 else 200
        r = leg_result(f"{name}_M{M}", leg2, leg2.time(steps, steps // 10, SECONDARY_REPLAYS), M, SECONDARY_REPLAYS)
        if M == 1:   # the streaming read of this leg's own bytes per launch
            sc = stream_leg(qgm, torch, leg2.wbytes, 200, 3, grids=(1024, 2048))["best"]
            r["stream_ceiling_GBps"] = sc["GBps"]
            r["frac_of_stream_ceiling"] = round(r["weight_GBps"] / sc["GBps"], 4)
        else:
            r["mfma_frac_derived_peak"] = round(r["TFLOPs"] / peaks["derived_TFLOPs"], 4)
            r["mfma_frac_sustained"] = round(r["TFLOPs"] / peaks["sustained_TFLOPs"], 4)
        if name == "prefill_int4_g128":
            r["traffic"] = load_traffic("gemm_int4_m128")
            r["dispatch_us"] = load_dispatch("gemm_int4_m128")
        secondary.append(r)
        del leg2
        torch.cuda.empty_cache()
    # same-buffer (cache-resident) rate of the headline case
    hot = Leg(qgm, torch, main_case, 1, min_bytes=0)
    secondary.append(dict(leg_result("decode_int4_g128_M1_cache_resident", hot, hot.time(400, 40, SECONDARY_REPLAYS), 1, SECONDARY_REPLAYS)))
    del hot
    secondary.append(loop_leg(qgm, torch, synth))
    secondary.append(loop_leg(qgm, torch, synth, M=1))
    secondary.append(fp16_leg(qgm, torch, synth, Ms=(1, 8, 128, 512)))

    achieved = wbytes / (ms * 1e-3) / 1e9
    traffic = load_traffic("gemv_int4_m1")
    ceiling = stream["best"]["GBps"]
    result = {
        "metric": "qGEMM weight GB/s at M=1, TFLOP/s at M=128, % of HBM/MFMA roofline",
        "value": round(achieved, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "ms_per_step_events": round(ms_events, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 (fp32 accumulation)",
        "data": "synthetic (seeded; W ~ N(0, 0.02) quantized, x ~ N(0, 1))",
        "config": {"workload": "decode GEMV, INT4 asymmetric g128, M=1, N=6144, K=2048",
                   "M": 1, "N": 6144, "K": 2048, "group": 128, "format": "int4_asym",
                   "weight_bytes_per_step": wbytes, "weight_copies": copies,
                   "weight_bytes_per_replay": wbytes * args.steps, "on_die_cache_bytes": MALL_BYTES,
                   "stamp_pair_ms": round(_STAMP_PAIR.get("ms", float("nan")), 6),
                   "timing": f"K steps captured in one HIP graph between two device clock stamps "
                             f"(qg_clock_stamp, stream order), after {WARM_STEPS} untimed steps on the last copies "
                             f"(the first kernel after the eviction pays about 2 us on its own); "
                             f"ms_per_step = (stamp span - the span of an "
                             f"empty stamp pair, stamp_pair_ms) / K, the median of "
                             f"{MAIN_REPLAYS} timed replays, each after a 512 MiB read that evicts the on-die cache; "
                             "ms_per_step_events = HIP events on the stream around the same replays, which also "
                             "hold the graph's own launch latency (events cannot be recorded inside a graph here)",
                   "replay_ms_per_step": [round(v, 6) for v in replay_ms]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "achieved_events": round(wbytes / (ms_events * 1e-3) / 1e9, 1),
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": gemv_kernel_name(qgm, main_case),
                     "algorithmic_bytes_per_launch": wbytes,
                     "achievable": ceiling,
                     "frac_of_achievable": round(achieved / ceiling, 4),
                     "achievable_kind": "plain streaming read of the same bytes per launch, same protocol",
                     "launch_floor_us": floor["us_per_launch"],
                     "dispatch_us": load_dispatch("gemv_int4_m1")},
        "ceilings": {"stream_read": stream, "empty_kernel": floor, "mfma": peaks},
        "secondary": secondary,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(synth, args.cpu_reps)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
