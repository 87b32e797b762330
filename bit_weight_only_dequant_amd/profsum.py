"""Summaries of the rocprofv3 runs of profile.sh: per-dispatch durations of
the benchmarked kernels and their HBM bytes (FETCH_SIZE / WRITE_SIZE scaled
by what the same counters read for a plain copy of known size), written as
the JSON files bench.py reads and as Markdown tables.

    python3 -m bit_weight_only_dequant_amd.profsum OUTDIR [--write DEST]

OUTDIR is the folder profile.sh filled; with --write the files go to DEST
(normally profiles/), else they are printed.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SRC = os.path.join(ROOT, "bit_weight_only_dequant_amd", "csrc", "kernels.hip")
COPY_BYTES = 512 << 20     # bench.py --only copy
GEMV_BYTES = 6684672       # INT4 g128 N=6144 K=2048: codes + scales + zeros
GEMM_BYTES = 8912896       # INT4 g128 N=8192 K=2048
PROFILE_CMD = "bash bit_weight_only_dequant_amd/profile.sh OUTDIR"
SUMMARY_CMD = "python3 -m bit_weight_only_dequant_amd.profsum OUTDIR --write profiles"


def kernel_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def _csv(outdir, run, suffix):
    files = sorted(glob.glob(os.path.join(outdir, run, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {os.path.join(outdir, run)}")
    out = []
    for f in files:
        with open(f, newline="") as fh:
            out += list(csv.DictReader(fh))
    return out


def trace(outdir, run):
    """(kernel name, duration ns) per dispatch, in dispatch order; the name
    carries the workgroup count when the trace has the grid columns."""
    rows = _csv(outdir, run, "kernel_trace.csv")
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    out = []
    for r in rows:
        name = r["Kernel_Name"]
        if r.get("Grid_Size_X") and r.get("Workgroup_Size_X"):
            wg = (int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))) * int(r.get("Grid_Size_Y") or 1)
            name = f"{name} [{wg} wg]"
        out.append((name, int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return out


def counter(outdir, run, name):
    """(kernel name, counter value) per dispatch, in dispatch order."""
    rows = [r for r in _csv(outdir, run, "counter_collection.csv") if r["Counter_Name"] == name]
    per = {}
    for r in rows:   # one row per dispatch for these derived counters; sum if split
        d = int(r["Dispatch_Id"])
        k, v = per.get(d, (r["Kernel_Name"], 0.0))
        per[d] = (k, v + float(r["Counter_Value"]))
    return [per[d] for d in sorted(per)]


def stats_us(durs_ns):
    v = np.asarray(durs_ns, dtype=np.float64) / 1e3
    return dict(n=int(v.size), avg=round(float(v.mean()), 3), p10=round(float(np.percentile(v, 10)), 3),
                p50=round(float(np.percentile(v, 50)), 3), p90=round(float(np.percentile(v, 90)), 3),
                min=round(float(v.min()), 3), max=round(float(v.max()), 3))


def select(items, key):
    return [v for k, v in items if key in k]


def calibration(outdir):
    f = select(counter(outdir, "pmc_copy_FETCH_SIZE", "FETCH_SIZE"), "copy")
    w = select(counter(outdir, "pmc_copy_WRITE_SIZE", "WRITE_SIZE"), "copy")
    fk, wk = float(np.median(f)), float(np.median(w))
    return dict(copy_bytes=COPY_BYTES, fetch_kib_per_copy=fk, write_kib_per_copy=wk,
                fetch_factor=round(COPY_BYTES / (fk * 1024), 4), write_factor=round(COPY_BYTES / (wk * 1024), 4),
                copies=len(f))


def kernel_bytes(outdir, leg, key, cal, algo):
    f = select(counter(outdir, f"pmc_{leg}_FETCH_SIZE", "FETCH_SIZE"), key)
    w = select(counter(outdir, f"pmc_{leg}_WRITE_SIZE", "WRITE_SIZE"), key)
    fb = float(np.median(f)) * 1024 * cal["fetch_factor"]
    wb = float(np.median(w)) * 1024 * cal["write_factor"]
    return dict(fetch_kib_median=round(float(np.median(f)), 1), write_kib_median=round(float(np.median(w)), 1),
                fetch_bytes=int(round(fb)), write_bytes=int(round(wb)), bytes=int(round(fb + wb)),
                algorithmic_weight_bytes=algo, ratio=round((fb + wb) / algo, 3), dispatches=len(f))


def loop_segments(outdir, run, name, L=8):
    """Per-dispatch values of counter `name` in the loop_prof run `run`, split
    at the evictions: (dispatches per loop k, the resident loops 1..L as an
    L x k array, the L loops that each follow an eviction as L x k).  Only the
    qGEMM kernels count, not the weight repack or torch's copies.  An
    eviction is a torch reduction over 512 MiB (the first one also fills its
    buffer and reads it twice); eviction kernels with no qGEMM dispatch
    between them are one boundary."""
    seq = counter(outdir, run, name)
    cur, segs = [], []
    after_evict = False
    for k, v in seq:
        if "reduce_kernel" in k or "FillFunctor" in k:
            if not after_evict:
                segs.append(cur)
                cur = []
            after_evict = True
        elif "qg::" in k and "pack" not in k:
            cur.append(v)
            after_evict = False
    segs.append(cur)
    k = len(segs[0])                 # dispatches per loop (the warm-up loop)
    if k == 0 or len(segs) != L + 2 or len(segs[1]) != L * k or any(len(x) != k for x in segs[2:]):
        raise ValueError(f"unexpected dispatch layout in {run}: {[len(x) for x in segs]}")
    return k, np.asarray(segs[1]).reshape(L, k), np.asarray(sum(segs[2:], [])).reshape(L, k)


def loop_bytes(outdir, leg, cal, L=8):
    """Per-loop calibrated FETCH_SIZE + WRITE_SIZE bytes of the loop_prof run:
    what the L2 reads from and writes to the fabric (Infinity Cache or HBM)."""
    k, fr, fc = loop_segments(outdir, f"pmc_{leg}_FETCH_SIZE", "FETCH_SIZE", L)
    _, wr, wc = loop_segments(outdir, f"pmc_{leg}_WRITE_SIZE", "WRITE_SIZE", L)
    res = ((fr * cal["fetch_factor"] + wr * cal["write_factor"]) * 1024).sum(axis=1)
    ctl = ((fc * cal["fetch_factor"] + wc * cal["write_factor"]) * 1024).sum(axis=1)
    return dict(dispatches_per_loop=k, resident_loop_bytes=[int(v) for v in res],
                loop1_bytes=int(res[0]), loops2_L_median_bytes=int(np.median(res[1:])),
                evict_each_loop_bytes=[int(v) for v in ctl], evict_each_loop_median_bytes=int(np.median(ctl)))


def loop_latency(outdir, leg, L=8):
    """Average latency (L2 cycles) of the L2's read requests to the fabric per
    loop, by Little's law: in-flight requests summed over cycles over the
    number of requests.  Reads the Infinity Cache serves return sooner than
    reads from HBM, so this tells the resident loops from the evicted ones."""
    _, lr, lc = loop_segments(outdir, f"pmc_{leg}_lat", "TCC_EA0_RDREQ_LEVEL_sum", L)
    _, qr, qc = loop_segments(outdir, f"pmc_{leg}_lat", "TCC_EA0_RDREQ_sum", L)
    res = lr.sum(axis=1) / qr.sum(axis=1)
    ctl = lc.sum(axis=1) / qc.sum(axis=1)
    return dict(resident_loop_latency_cycles=[round(float(v), 1) for v in res],
                loop1_latency_cycles=round(float(res[0]), 1),
                loops2_L_median_latency_cycles=round(float(np.median(res[1:])), 1),
                evict_each_loop_latency_cycles=[round(float(v), 1) for v in ctl],
                evict_each_loop_median_latency_cycles=round(float(np.median(ctl)), 1),
                read_requests_per_loop=int(np.median(qr.sum(axis=1))))


def persistent_residency(outdir, cal, L=8, reps=3):
    """The one-launch persistent block (loop_prof_persistent): `reps` launches
    of one loop, then `reps` of L loops, each after an eviction.  Per launch:
    calibrated fabric bytes and the L2-miss latency; per loop of the L-loop
    launch, bytes / L."""
    def per_launch(run, name):
        v = select(counter(outdir, run, name), "loop_block_kernel")
        if len(v) != 2 * reps:
            raise ValueError(f"{run}: {len(v)} launches of the persistent kernel, expected {2 * reps}")
        return np.asarray(v, dtype=np.float64)
    f = per_launch("pmc_persist_FETCH_SIZE", "FETCH_SIZE") * 1024 * cal["fetch_factor"]
    w = per_launch("pmc_persist_WRITE_SIZE", "WRITE_SIZE") * 1024 * cal["write_factor"]
    lev = per_launch("pmc_persist_lat", "TCC_EA0_RDREQ_LEVEL_sum")
    req = per_launch("pmc_persist_lat", "TCC_EA0_RDREQ_sum")
    b1, bL = float(np.median((f + w)[:reps])), float(np.median((f + w)[reps:]))
    l1, lL = float(np.median((lev / req)[:reps])), float(np.median((lev / req)[reps:]))
    return dict(launch_1_loop_bytes=int(b1), launch_L_loops_bytes=int(bL), L=L,
                bytes_per_loop_L_launch=int(bL / L), latency_1_loop_cycles=round(l1, 1),
                latency_L_loops_cycles=round(lL, 1))


def plain_step_us(outdir, leg):
    """us per step of `bench.py --only leg` run without the profiler on the
    same machine (profile.sh runs it first), or None when it is absent."""
    try:
        lines = open(os.path.join(outdir, f"plain_{leg}.json")).read().strip().splitlines()
        r = json.loads(lines[-1])
    except Exception:
        return None
    return r.get("us_per_call", r.get("us_per_launch"))


def plain_note(step_us, avg_us, what):
    if step_us is None:
        return ""
    return (f"  Without the profiler, on the same machine just before (`bench.py --only {what}`, device clock "
            f"stamps inside the graph), one step takes {step_us} us; the traced average is {avg_us} us.")


def md_trace(title, cmd_note, rows):
    out = [f"# {title}", "", "Commands (GPU host, repository root):", "", "```", PROFILE_CMD, SUMMARY_CMD, "```", "",
           cmd_note, "", "| kernel | dispatches | avg us | p10 | p50 | p90 | min | max |", "|---|---|---|---|---|---|---|---|"]
    for name, s in rows:
        out.append(f"| {name} | {s['n']} | {s['avg']} | {s['p10']} | {s['p50']} | {s['p90']} | {s['min']} | {s['max']} |")
    return "\n".join(out) + "\n"


def short(name):
    """Kernel name without its parameter list, keeping the workgroup count."""
    base, _, grid = name.partition(" [")
    base = base.replace("void ", "").replace("(anonymous namespace)::", "")
    if "(" in base:
        base = base[:base.index("(")]
    return base + (f" [{grid}" if grid else "")


def per_kernel(items):
    names = []
    for k, _ in items:
        if "qg::" in k and k not in names:
            names.append(k)
    return [(short(n), stats_us([d for k, d in items if k == n])) for n in names]


VALU_COUNTERS = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_LDS", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
                 "SQ_WAVE_CYCLES")


def valu_counters(outdir, run, key):
    """Medians over the GEMV dispatches of the SQ counters of `run`, and the
    same per wave."""
    med = {c: float(np.median(select(counter(outdir, run, c), key))) for c in VALU_COUNTERS}
    n = len(select(counter(outdir, run, "SQ_WAVES"), key))
    waves = med["SQ_WAVES"]
    per = {c: round(med[c] / waves, 1) for c in VALU_COUNTERS if c != "SQ_WAVES"}
    return dict(dispatches=n, median=med, per_wave=per,
                wait_share=round(med["SQ_WAIT_ANY"] / med["SQ_WAVE_CYCLES"], 3),
                issue_wait_share=round(med["SQ_WAIT_INST_ANY"] / med["SQ_WAVE_CYCLES"], 3))


def valu_file(outdir, sha):
    rows = []
    for label, run, chunks in (("INT4 g128, M=1, N=6144, K=2048 (decode)", "pmc_main_valu", 6144 * 2048 // 32),
                               ("INT2 g64, M=1, N=8192, K=2048", "pmc_int2_valu", 8192 * 2048 // 64)):
        v = valu_counters(outdir, run, "gemv")
        m, pw = v["median"], v["per_wave"]
        rows.append(f"| {label} | {v['dispatches']} | {m['SQ_WAVES']:.0f} | {pw['SQ_INSTS_VALU']} | "
                    f"{m['SQ_INSTS_VALU'] * 64 / chunks:.1f} | {pw['SQ_INSTS_VMEM_RD']} | {pw['SQ_INSTS_LDS']} | "
                    f"{v['wait_share']} | {v['issue_wait_share']} |")
    return "\n".join([
        "# Instruction counters: the M = 1 GEMVs (rocprofv3 --pmc, per dispatch)", "",
        "Commands (GPU host, repository root):", "", "```", "bash bit_weight_only_dequant_amd/profile.sh OUTDIR valu",
        "python3 -m bit_weight_only_dequant_amd.profsum OUTDIR --part valu --write profiles", "```", "",
        f"Runs `pmc_main_valu` (`rocprofv3 --pmc {' '.join(VALU_COUNTERS)} -- python3 bench.py --only main "
        f"--steps 81 --warmup 8`) and `pmc_int2_valu` (the same counters, `--only int2 --steps 103 --warmup 8`).  "
        f"Kernel sources sha256[:16] = `{sha}`; medians over the GEMV dispatches.  A chunk is one lane's "
        f"16-byte code load (32 INT4 or 64 INT2 codes); VALU per chunk = the VALU instructions one lane issues "
        f"per chunk it dequantizes (SQ_INSTS_VALU counts wave instructions: x 64 lanes / chunks per launch), "
        f"with the staging, lane sums and epilogue included; waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES, the "
        f"share of a wave's life spent waiting (loads in flight, LDS, barriers); issue waits = "
        f"SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES, the share spent ready but waiting for an instruction to issue.",
        "", "| launch | dispatches | waves | VALU per wave | VALU per chunk | vector-memory reads per wave | "
        "LDS instructions per wave | waiting | issue waits |", "|---|---|---|---|---|---|---|---|---|", *rows,
        ""]) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("outdir")
    ap.add_argument("--write", default=None)
    ap.add_argument("--part", choices=["all", "valu"], default="all",
                    help="valu: only the instruction counters of the M = 1 GEMVs (profile.sh OUTDIR valu)")
    a = ap.parse_args()
    sha = kernel_hash()
    files = {}
    files["gemv_m1_valu_counters.md"] = valu_file(a.outdir, sha)
    if a.part == "valu":
        write_files(files, a.write)
        return 0

    tm = trace(a.outdir, "trace_main")
    tg = trace(a.outdir, "trace_gemm")
    ts = trace(a.outdir, "trace_stream")
    tf = trace(a.outdir, "trace_floor")
    gemv = stats_us(select(tm, "gemv"))
    gemm = stats_us(select(tg, "gemm_kernel"))
    empty = stats_us(select(tf, "empty_kernel"))
    p_main, p_gemm, p_floor = (plain_step_us(a.outdir, leg) for leg in ("main", "gemm", "floor"))
    for st, p in ((gemv, p_main), (gemm, p_gemm), (empty, p_floor)):
        if p is not None:
            st["bench_step_us_same_machine"] = p
    files["dispatch.json"] = json.dumps(dict(kernel_src_sha=sha, gemv_int4_m1=gemv, gemm_int4_m128=gemm,
                                             empty_kernel=empty), indent=1) + "\n"
    files["empty_kernel_launch_floor_kernel_trace.md"] = md_trace(
        "Kernel trace: the empty kernel of the decode GEMV's grid (768 x 512), graph-replayed",
        "Run `trace_floor` (`... -- python3 bench.py --only floor`): bench.py times the same graph at its "
        "launch floor per step; the traced duration of each dispatch also carries what the profiler adds "
        "to every dispatch, the same for every kernel of the other traces." +
        plain_note(p_floor, empty["avg"], "floor") +
        ("  The difference is the tracer's own cost per dispatch on this machine; it weighs most on the "
         "shortest kernels." if p_floor is not None else ""),
        [(short(n), stats_us([d for k, d in tf if k == n])) for n in dict.fromkeys(k for k, _ in tf)
         if "empty_kernel" in n])
    files["gemv_int4_g128_m1_n6144_k2048_kernel_trace.md"] = md_trace(
        "Kernel trace: decode GEMV, INT4 g128, M=1, N=6144, K=2048",
        f"Run `trace_main` (`rocprofv3 --kernel-trace --stats -- python3 bench.py --only main`): every dispatch "
        f"of the headline leg (warm-up, graph upload and the timed replays; the cache is evicted before each "
        f"timed replay).  Kernel sources sha256[:16] = `{sha}`.  Algorithmic bytes per launch {GEMV_BYTES}: "
        f"{GEMV_BYTES / (gemv['avg'] * 1e3):.1f} GB/s at the average duration." +
        plain_note(p_main, gemv["avg"], "main"), per_kernel(tm))
    files["gemm_int4_g128_m128_n8192_k2048_kernel_trace.md"] = md_trace(
        "Kernel trace: prefill GEMM, INT4 g128, M=128, N=8192, K=2048",
        f"Run `trace_gemm` (`... -- python3 bench.py --only gemm`).  Kernel sources sha256[:16] = `{sha}`.  "
        f"2*M*N*K = {2 * 128 * 8192 * 2048} flops per launch: "
        f"{2 * 128 * 8192 * 2048 / (gemm['avg'] * 1e3) / 1e3:.1f} TFLOP/s at the average duration." +
        plain_note(p_gemm, gemm["avg"], "gemm"), per_kernel(tg))
    files["stream_read_6684672B_kernel_trace.md"] = md_trace(
        "Kernel trace: streaming read of 6684672 bytes per launch (the decode weight bytes)",
        f"Run `trace_stream` (`... -- python3 bench.py --only stream`): four grids (256, 512, 1024, 2048 "
        f"workgroups) in turn; one row per grid.",
        [(short(n), stats_us([d for k, d in ts if k == n])) for n in dict.fromkeys(k for k, _ in ts)
         if "stream_read" in n])
    for m, run in ((128, "trace_loop128"), (1, "trace_loop1")):
        tl = trace(a.outdir, run)
        files[f"loop_block_int4_g128_m{m}_d2048_f8192_kernel_trace.md"] = md_trace(
            f"Kernel trace: looped shared block, INT4 g128, M={m}, D=2048, F=8192, L=8",
            f"Run `{run}` (`... -- python3 bench.py --only loop --loop-m {m}`): the block resident (cache "
            f"evicted before loop 1), warm, and with the cache evicted before every loop.  Kernel sources "
            f"sha256[:16] = `{sha}`.", per_kernel(tl))

    cal = calibration(a.outdir)
    t_gemv = kernel_bytes(a.outdir, "main", "gemv", cal, GEMV_BYTES)
    t_gemm = kernel_bytes(a.outdir, "gemm", "gemm_kernel", cal, GEMM_BYTES)
    files["traffic.json"] = json.dumps(dict(kernel_src_sha=sha, calibration=cal, gemv_int4_m1=t_gemv,
                                            gemm_int4_m128=t_gemm), indent=1) + "\n"
    lm = {}
    for m, leg, name in ((128, "loop128", "loop_block_int4_g128"), (1, "loop1", "loop_block_int4_g128_M1")):
        lm[name] = loop_bytes(a.outdir, leg, cal)
        lm[name].update(loop_latency(a.outdir, leg))
        lm[name]["weight_bytes_per_loop"] = 26738688
    pr = persistent_residency(a.outdir, cal)
    lm["loop_block_int4_g128_M1"]["one_launch"] = pr
    files["loop_traffic.json"] = json.dumps(dict(kernel_src_sha=sha, calibration=cal, **lm), indent=1) + "\n"

    hdr = ["Commands (GPU host, repository root):", "", "```", PROFILE_CMD, SUMMARY_CMD, "```", "",
           f"Kernel sources sha256[:16] = `{sha}` (bench.py reports these bytes only while kernels.hip has "
           f"this hash).", "",
           f"Calibration: a plain device copy of 512 MiB (`bench.py --only copy`, torch `copy_`) reads "
           f"FETCH_SIZE = {cal['fetch_kib_per_copy']:.1f} KiB and WRITE_SIZE = {cal['write_kib_per_copy']:.1f} "
           f"KiB per dispatch, so bytes = FETCH_SIZE x {cal['fetch_factor']} x 1024 and WRITE_SIZE x "
           f"{cal['write_factor']} x 1024.", ""]
    t = ["# HBM traffic counters (rocprofv3 --pmc), per dispatch", ""] + hdr + [
        "| kernel | dispatches | FETCH_SIZE KiB (median) | WRITE_SIZE KiB (median) | calibrated bytes | "
        "algorithmic weight bytes | ratio |", "|---|---|---|---|---|---|---|",
        f"| GEMV (M=1, N=6144, K=2048, INT4 g128) | {t_gemv['dispatches']} | {t_gemv['fetch_kib_median']} | "
        f"{t_gemv['write_kib_median']} | {t_gemv['bytes']} | {GEMV_BYTES} | {t_gemv['ratio']} |",
        f"| GEMM (M=128, N=8192, K=2048, INT4 g128) | {t_gemm['dispatches']} | {t_gemm['fetch_kib_median']} | "
        f"{t_gemm['write_kib_median']} | {t_gemm['bytes']} | {GEMM_BYTES} | {t_gemm['ratio']} |", "",
        "FETCH_SIZE counts what the L2s request from the fabric (Infinity Cache or HBM).  Expected with each "
        "byte of W fetched once: GEMV W 6684672 + x 4096 per XCD x 8 = 6717440 B read, y 12288 B written; GEMM W "
        f"{GEMM_BYTES} + x 524288 per XCD x 8 (every column tile reads all of x, and each XCD's L2 fetches its "
        f"own copy) = {GEMM_BYTES + 8 * 524288} B read, y 2097152 B written.  Measured reads: GEMV "
        f"{t_gemv['fetch_bytes']} B, GEMM {t_gemm['fetch_bytes']} B.", ""]
    files["hbm_traffic_counters.md"] = "\n".join(t) + "\n"
    lt = ["# Looped shared block: L2 fabric bytes and L2-miss latency per loop (rocprofv3 --pmc)", ""] + hdr + [
        "Runs `pmc_loop128_*` / `pmc_loop1_*` (`bench.py --only loop_prof`): the warm-up loop, an eviction, L=8 "
        "loops back to back (loop 1 cold, loops 2..8 find the shared weights where loop 1 left them), then 8 "
        "single loops each after an eviction (the control).  Per loop, over its qGEMM dispatches:", "",
        "- bytes = calibrated FETCH_SIZE + WRITE_SIZE: what the L2s read from and write to the fabric.  The "
        "L2s keep nothing from one kernel to the next, so this is the same in every loop; whether the "
        "Infinity Cache (256 MB, behind the L2s) or HBM serves those reads the counter cannot tell;",
        "- latency = TCC_EA0_RDREQ_LEVEL_sum / TCC_EA0_RDREQ_sum (run `pmc_loop*_lat`): the average time, in "
        "L2 cycles, that the L2's read requests to the fabric are in flight.  Reads the Infinity Cache "
        "serves return sooner than reads from HBM, so the resident loops against the control show where "
        "the shared weights are read from.", "",
        "The shared weights are 26738688 bytes per loop.", "",
        "| block | dispatches per loop | bytes loop 1 | bytes loops 2..8 (median) | bytes, evicted before every "
        "loop (median) | latency loop 1 | latency loops 2..8 (median) | latency, evicted before every loop "
        "(median) |", "|---|---|---|---|---|---|---|---|"]
    for name, v in lm.items():
        lt.append(f"| {name} | {v['dispatches_per_loop']} | {v['loop1_bytes']} | {v['loops2_L_median_bytes']} | "
                  f"{v['evict_each_loop_median_bytes']} | {v['loop1_latency_cycles']} | "
                  f"{v['loops2_L_median_latency_cycles']} | {v['evict_each_loop_median_latency_cycles']} |")
    lt += ["", "The M = 1 block as one persistent launch for all L = 8 loops (`qloop_block_persistent` mode 1; runs "
           "`pmc_persist_*`, `bench.py --only loop_prof_persistent`: three launches of one loop, then three of eight, "
           "each after an eviction).  The workgroup that runs a block of rows runs it in every loop, and nothing "
           "invalidates the L2s between loops inside one launch, so each XCD's L2 can keep its rows' weights:", "",
           "| launch | fabric bytes per launch | per loop | L2-miss latency (cycles) |", "|---|---|---|---|",
           f"| 1 loop | {pr['launch_1_loop_bytes']} | {pr['launch_1_loop_bytes']} | {pr['latency_1_loop_cycles']} |",
           f"| 8 loops | {pr['launch_L_loops_bytes']} | {pr['bytes_per_loop_L_launch']} | "
           f"{pr['latency_L_loops_cycles']} |"]
    lt += ["", "Latency of each loop (resident run, loops 1..8; then the control):", ""]
    for name, v in lm.items():
        lt.append(f"- {name}: {v['resident_loop_latency_cycles']}; control {v['evict_each_loop_latency_cycles']}")
    files["loop_block_int4_g128_traffic.md"] = "\n".join(lt) + "\n"

    mc = {}
    for name in ("SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"):
        mc[name] = float(np.median(select(counter(a.outdir, "pmc_gemm_mfma", name), "gemm_kernel")))
    flops = 2 * 128 * 8192 * 2048
    cycles = gemm["avg"] * 1e-6 * 2.4e9
    busy = mc["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * cycles)
    files["gemm_int4_g128_m128_n8192_k2048_mfma_counters.md"] = "\n".join([
        "# MFMA counters: prefill GEMM, INT4 g128, M=128, N=8192, K=2048 (rocprofv3 --pmc, per dispatch)", "",
        "Commands (GPU host, repository root):", "", "```", PROFILE_CMD, SUMMARY_CMD, "```", "",
        f"Run `pmc_gemm_mfma` (`rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES "
        f"GRBM_GUI_ACTIVE -- python3 bench.py --only gemm --steps 64 --warmup 8`).  Kernel sources sha256[:16] = "
        f"`{sha}`; medians over the GEMM dispatches:", "",
        "| counter | value | reading |", "|---|---|---|",
        f"| SQ_INSTS_VALU_MFMA_MOPS_F16 | {mc['SQ_INSTS_VALU_MFMA_MOPS_F16']:.0f} | x 512 = "
        f"{mc['SQ_INSTS_VALU_MFMA_MOPS_F16'] * 512:.4g} FLOP; 2*M*N*K = {flops:.4g} |",
        f"| SQ_VALU_MFMA_BUSY_CYCLES | {mc['SQ_VALU_MFMA_BUSY_CYCLES']:.0f} | busy SIMD-cycles |",
        f"| SQ_BUSY_CYCLES | {mc['SQ_BUSY_CYCLES']:.0f} | |",
        f"| GRBM_GUI_ACTIVE | {mc['GRBM_GUI_ACTIVE']:.0f} | summed over the 8 XCDs |", "",
        f"MFMA busy share = busy SIMD-cycles / (1024 SIMDs x the kernel's average duration in cycles at 2.4 GHz, "
        f"{gemm['avg']} us from `trace_gemm`) = {100 * busy:.1f} %.", ""]) + "\n"

    write_files(files, a.write)
    return 0


def write_files(files, dest):
    if dest:
        os.makedirs(dest, exist_ok=True)
        for n, txt in files.items():
            open(os.path.join(dest, n), "w").write(txt)
            print("wrote", os.path.join(dest, n))
    else:
        for n, txt in files.items():
            print(f"---- {n}\n{txt}")


if __name__ == "__main__":
    sys.exit(main())
