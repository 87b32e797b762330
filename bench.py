"""Benchmark of the weight-only low-bit matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only main]

A step is one qgemm call of the decode workload: INT4 asymmetric, group 128,
M=1, N=6144, K=2048 (the fused QKV of a D=2048 block).  Each step reads a
different copy of the packed weight, scales and zero points; the copies add
up to more than twice the 256 MB on-die cache, so every step streams its
weight bytes from HBM.  The K timed steps are captured once in a HIP graph and
replayed, bracketed by events on the stream the kernels run on.

One JSON line is printed: value = weight GB/s at M=1, plus the roofline of the
GEMV kernel, the CPU oracle timed on the host, and secondary legs (M=8, the
M=128 MFMA GEMM in TFLOP/s, INT2 and q4_0, the looped shared block).
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SRC = os.path.join(ROOT, "bit_weight_only_dequant_amd", "csrc", "kernels.hip")


def kernel_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=810)
    ap.add_argument("--warmup", type=int, default=81)
    ap.add_argument("--only", choices=["all", "main", "gemm", "loop", "fp16", "copy"], default="all",
                    help="main/gemm/loop/fp16: run one leg (for profiler runs); copy: the calibration copy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
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
        """ms per step: one timed replay of a graph of `steps` calls, or the
        median over `replays` timed replays of it (secondary legs: a single
        replay of a ~2 ms graph varies by up to 10 % at M = 128)."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                self.step(i)
        g.replay()  # first replay uploads the graph; not timed
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        stream = torch.cuda.current_stream()
        times = []
        for _ in range(replays):
            start.record(stream)
            g.replay()
            stop.record(stream)
            stop.synchronize()
            times.append(start.elapsed_time(stop) / steps)
        return sorted(times)[len(times) // 2]


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


def cpu_baseline(case, M, seconds):
    """The oracle as it stands, on a bounded sample of the decode workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    x = case.x[:M]
    calls = 0
    t0 = time.perf_counter()
    while True:
        oracle.qgemm_ref(x, case.words, case.scales, case.zeros, M, case.N, case.K, case.group, case.fmt)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    wbytes = case.weight_bytes
    return dict(value=round(wbytes * calls / el / 1e9, 4), unit="GB/s", cores=int(blas_threads),
                kind="oracle",
                sample=f"{calls} oracle calls (unpack, fp32 dequant, fp64 product) on the decode "
                       f"workload M={M} N={case.N} K={case.K} INT4 g{case.group}, {el:.1f} s; "
                       f"elementwise steps single-threaded, BLAS with {blas_threads} threads")


def loop_leg(qgm, torch, synth, L=8, flush=True, M=128):
    """Looped shared block: per-loop time, cold (on-die cache flushed) vs warm.
    M = 128 is the prefill-sized block; M = 1 the decode step (GEMV kernels)."""
    lc = synth.loop_workload(M=M, L=L)
    lins = [qgm.QuantLinear.from_case(c, "cuda") for c in lc.linears()]
    x0 = qgm.to_half_tensor(lc.x0, "cuda")
    M, D = lc.x0.shape
    F = lc.up.N
    scratch = torch.empty(M * (3 * D + D + F), dtype=torch.float16, device="cuda")
    x = x0.clone()
    qgm.loop_block(x, lins, L, scratch=scratch)  # warm-up, allocates the workspace
    torch.cuda.synchronize()
    flush_buf = torch.empty(2 * MALL_BYTES // 2, dtype=torch.float16, device="cuda")
    res = {}
    for mode in ("cold", "warm"):
        x.copy_(x0)
        if mode == "cold":
            flush_buf.fill_(1.0)  # evicts the weights from the on-die cache
        else:
            qgm.loop_block(x, lins, 1, scratch=scratch)
            x.copy_(x0)
        events = [torch.cuda.Event(enable_timing=True) for _ in range(L + 1)]
        qgm.loop_block(x, lins, L, scratch=scratch, events=events)
        events[-1].synchronize()
        per = [events[i].elapsed_time(events[i + 1]) for i in range(L)]
        res[mode] = per
    wbytes = sum(l.weight_bytes for l in lins)
    flops = 2.0 * M * (D * 3 * D + D * D + D * F + F * D)
    cold, warm = res["cold"], res["warm"]
    return dict(leg="loop_block_int4_g128" + ("" if M == 128 else f"_M{M}"), M=M, D=D, F=F, L=L,
                weight_bytes_per_loop=wbytes,
                cold_loop_ms=[round(v, 4) for v in cold], warm_loop_ms=[round(v, 4) for v in warm],
                loop1_cold_ms=round(cold[0], 4),
                loops2_L_ms=round(float(np.median(cold[1:])), 4),   # median: robust to launch jitter
                TFLOPs_loops2_L=round(flops / (float(np.median(cold[1:])) * 1e-3) / 1e12, 2),
                weight_GBps_loop1_cold=round(wbytes / (cold[0] * 1e-3) / 1e9, 1))


def graph_time(torch, step, steps, warmup):
    """ms per step of `step(i)`, captured once in a HIP graph and replayed."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    start.record(stream)
    g.replay()
    stop.record(stream)
    stop.synchronize()
    return start.elapsed_time(stop) / steps


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

        t_deq = graph_time(torch, deq_step, steps, 10)
        t_f16 = graph_time(torch, f16_step, steps, 10)
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
    out = {}
    if args.only in ("all", "main"):
        leg = Leg(qgm, torch, main_case, 1)
        ms = leg.time(args.steps, args.warmup)
        main_r = leg_result("decode_int4_g128_M1", leg, ms, 1)
        out["main"] = (leg, ms, main_r)
        if args.only == "main":
            print(json.dumps(main_r), flush=True)
            return
    if args.only == "gemm":
        c = synth.workload("prefill_int4_g128")
        leg = Leg(qgm, torch, c, 128)
        ms = leg.time(max(64, args.steps // 8), 8, replays=SECONDARY_REPLAYS)
        print(json.dumps(leg_result("prefill_int4_g128_M128", leg, ms, 128, SECONDARY_REPLAYS)), flush=True)
        return
    if args.only == "loop":
        print(json.dumps(loop_leg(qgm, torch, synth)), flush=True)
        return
    if args.only == "fp16":
        print(json.dumps(fp16_leg(qgm, torch, synth)), flush=True)
        return

    secondary = []
    leg8 = Leg(qgm, torch, main_case, 8)
    secondary.append(leg_result("decode_int4_g128_M8", leg8, leg8.time(400, 40, SECONDARY_REPLAYS), 8, SECONDARY_REPLAYS))
    del leg8
    for name, M in (("prefill_int4_g128", 128), ("int2_g64", 1), ("int2_g64", 128),
                    ("q4_0_b32", 1), ("q4_0_b32", 128), ("q8_0_b32", 1), ("q8_0_b32", 128),
                    ("q4k_s256", 1), ("q4k_s256", 128)):
        c = synth.workload(name)
        leg = Leg(qgm, torch, c, M)
        steps = 400 if M == 1 else 200
        secondary.append(leg_result(f"{name}_M{M}", leg, leg.time(steps, steps // 10, SECONDARY_REPLAYS), M, SECONDARY_REPLAYS))
        del leg
        torch.cuda.empty_cache()
    # same-buffer (cache-resident) rate of the headline case
    hot = Leg(qgm, torch, main_case, 1, min_bytes=0)
    secondary.append(dict(leg_result("decode_int4_g128_M1_cache_resident", hot, hot.time(400, 40, SECONDARY_REPLAYS), 1, SECONDARY_REPLAYS)))
    del hot
    secondary.append(loop_leg(qgm, torch, synth))
    secondary.append(loop_leg(qgm, torch, synth, M=1))
    secondary.append(fp16_leg(qgm, torch, synth, Ms=(1, 8, 128, 512)))

    leg, ms, main_r = out["main"]
    wbytes = leg.wbytes
    achieved = wbytes / (ms * 1e-3) / 1e9
    traffic = load_traffic("gemv_int4_m1")
    result = {
        "metric": "qGEMM weight GB/s at M=1, TFLOP/s at M=128, % of HBM/MFMA roofline",
        "value": round(achieved, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 (fp32 accumulation)",
        "data": "synthetic (seeded; W ~ N(0, 0.02) quantized, x ~ N(0, 1))",
        "config": {"workload": "decode GEMV, INT4 asymmetric g128, M=1, N=6144, K=2048",
                   "M": 1, "N": 6144, "K": 2048, "group": 128, "format": "int4_asym",
                   "weight_bytes_per_step": wbytes, "weight_copies": leg.copies,
                   "timing": "K steps captured in one HIP graph, replayed once between events"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": gemv_kernel_name(qgm, main_case),
                     "algorithmic_bytes_per_launch": wbytes},
        "secondary": secondary,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(main_case, 1, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
