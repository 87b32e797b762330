"""The rocprofv3 summarizer on fabricated CSV files (no GPU): calibration
against the plain copy, per-kernel medians, and the split of the looped
block's dispatches into resident and evict-every-loop loops."""
import csv
import json
import os

import numpy as np
import pytest

from bit_weight_only_dequant_amd import profsum

TRACE_COLS = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
PMC_COLS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
FILL = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<c10::Half> >"
COPY = "void at::native::direct_copy_kernel_cuda(at::TensorIteratorBase&)"
GEMM = "void qg::gemm_kernel<0, 4, 4, 8, 2, 4>(qg::GemmArgs)"
GEMV = "void qg::gemv_half_kernel<0, 8, 2, 1>(qg::GemvArgs)"
PACK = "qg::qpack_kernel(unsigned int const*, unsigned int*, int, int, int, int, long)"
REDUCE = "void at::native::reduce_kernel<512, 1, at::native::ReduceOp<c10::Half, at::native::func_wrapper_t<float> > >"
ZERO = "__amd_rocclr_fillBufferAligned"


def write(path, cols, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def pmc(outdir, run, counter, seq):
    rows = [dict(Dispatch_Id=i + 1, Kernel_Name=k, Counter_Name=counter, Counter_Value=v)
            for i, (k, v) in enumerate(seq)]
    write(os.path.join(outdir, run, "host", "1", f"{run}_counter_collection.csv"), PMC_COLS, rows)


def trace(outdir, run, seq):
    rows, t = [], 1000
    for i, (k, d) in enumerate(seq):
        rows.append(dict(Kind="KERNEL_DISPATCH", Dispatch_Id=i + 1, Kernel_Name=k, Start_Timestamp=t,
                         End_Timestamp=t + d))
        t += d + 500
    write(os.path.join(outdir, run, "host", "1", f"{run}_kernel_trace.csv"), TRACE_COLS, rows)


def test_calibration_and_kernel_bytes(tmp_path):
    out = str(tmp_path)
    kib = profsum.COPY_BYTES / 1024
    pmc(out, "pmc_copy_FETCH_SIZE", "FETCH_SIZE", [(FILL, 0.0)] + [(COPY, kib / 2)] * 3)
    pmc(out, "pmc_copy_WRITE_SIZE", "WRITE_SIZE", [(FILL, kib)] + [(COPY, kib)] * 3)
    cal = profsum.calibration(out)
    assert cal["fetch_factor"] == 2.0 and cal["write_factor"] == 1.0 and cal["copies"] == 3
    pmc(out, "pmc_gemm_FETCH_SIZE", "FETCH_SIZE", [(PACK, 99.0), (GEMM, 4000.0), (GEMM, 5000.0), (GEMM, 6000.0)])
    pmc(out, "pmc_gemm_WRITE_SIZE", "WRITE_SIZE", [(PACK, 99.0), (GEMM, 2048.0), (GEMM, 2048.0), (GEMM, 2048.0)])
    t = profsum.kernel_bytes(out, "gemm", "gemm_kernel", cal, profsum.GEMM_BYTES)
    assert t["dispatches"] == 3
    assert t["bytes"] == 5000 * 1024 * 2 + 2048 * 1024


def test_loop_split(tmp_path):
    out = str(tmp_path)
    cal = dict(fetch_factor=2.0, write_factor=1.0)
    L, k = 8, 4
    # repack kernels, the warm-up loop, eviction, L resident loops, then L x (eviction, one loop)
    fetch = [(PACK, 1.0)] * 4 + [(GEMM, 10.0)] * k + [(COPY, 50.0), (FILL, 0.0)]
    for i in range(L):
        fetch += [(GEMM, 100.0 if i == 0 else 3.0)] * k
    fetch.append((COPY, 50.0))
    for i in range(L):
        fetch += [(FILL, 0.0)] + [(GEMM, 100.0)] * k
    write_seq = [(kname, 0.5 if "qg::gemm" in kname else 7.0) for kname, _ in fetch]
    pmc(out, "pmc_loop128_FETCH_SIZE", "FETCH_SIZE", fetch)
    pmc(out, "pmc_loop128_WRITE_SIZE", "WRITE_SIZE", write_seq)
    r = profsum.loop_bytes(out, "loop128", cal, L=L)
    per = lambda f: k * (f * 1024 * 2 + 0.5 * 1024)
    assert r["dispatches_per_loop"] == k
    assert r["loop1_bytes"] == int(per(100.0))
    assert r["loops2_L_median_bytes"] == int(per(3.0))
    assert r["evict_each_loop_bytes"] == [int(per(100.0))] * L


def test_loop_latency(tmp_path):
    out = str(tmp_path)
    L, k = 8, 4
    lev, req = [(GEMM, 1.0)] * k + [(FILL, 0.0)], [(GEMM, 1.0)] * k + [(FILL, 0.0)]
    for i in range(L):   # resident: 200 cycles in loops 2..8, 900 in loop 1
        lev += [(GEMM, (900.0 if i == 0 else 200.0) * 10)] * k
        req += [(GEMM, 10.0)] * k
    for i in range(L):   # control: 800 cycles
        lev += [(FILL, 0.0)] + [(GEMM, 8000.0)] * k
        req += [(FILL, 0.0)] + [(GEMM, 10.0)] * k
    rows = [dict(Dispatch_Id=i + 1, Kernel_Name=kn, Counter_Name=c, Counter_Value=v)
            for c, seq in (("TCC_EA0_RDREQ_LEVEL_sum", lev), ("TCC_EA0_RDREQ_sum", req))
            for i, (kn, v) in enumerate(seq)]
    write(os.path.join(out, "pmc_loop1_lat", "h", "1", "x_counter_collection.csv"), PMC_COLS, rows)
    r = profsum.loop_latency(out, "loop1", L=L)
    assert r["loop1_latency_cycles"] == 900.0
    assert r["loops2_L_median_latency_cycles"] == 200.0
    assert r["evict_each_loop_median_latency_cycles"] == 800.0


def test_loop_split_rejects_a_bad_layout(tmp_path):
    out = str(tmp_path)
    seq = [(GEMM, 1.0)] * 4 + [(FILL, 0.0)] + [(GEMM, 1.0)] * 5
    pmc(out, "pmc_x_FETCH_SIZE", "FETCH_SIZE", seq)
    pmc(out, "pmc_x_WRITE_SIZE", "WRITE_SIZE", seq)
    with pytest.raises(ValueError):
        profsum.loop_bytes(out, "x", dict(fetch_factor=1.0, write_factor=1.0), L=8)


def test_trace_stats(tmp_path):
    out = str(tmp_path)
    durs = list(range(1000, 11000, 1000))   # 1..10 us
    trace(out, "trace_main", [(PACK, 5)] + [(GEMV, d) for d in durs])
    items = profsum.trace(out, "trace_main")
    s = profsum.stats_us(profsum.select(items, "gemv"))
    assert s["n"] == 10 and s["avg"] == 5.5 and s["min"] == 1.0 and s["max"] == 10.0
    assert s["p50"] == pytest.approx(float(np.percentile(np.arange(1, 11), 50)))


def test_loop_split_at_read_evictions(tmp_path):
    # the eviction is a reduction over 512 MiB; its first call also fills the
    # buffer and reads it twice: one boundary, however many kernels
    out = str(tmp_path)
    cal = dict(fetch_factor=2.0, write_factor=1.0)
    L, k = 8, 4
    setup = [(FILL, 0.0)] + [(ZERO, 0.0), (REDUCE, 9.0)] * 3
    fetch = [(PACK, 1.0)] * 4 + [(GEMM, 10.0)] * k + [(COPY, 50.0)] + setup
    for i in range(L):
        fetch += [(GEMM, 100.0 if i == 0 else 3.0)] * k
    for i in range(L):
        fetch += [(COPY, 50.0), (ZERO, 0.0), (REDUCE, 9.0)] + [(GEMM, 100.0)] * k
    write_seq = [(kname, 0.5 if "qg::gemm" in kname else 7.0) for kname, _ in fetch]
    pmc(out, "pmc_loop1_FETCH_SIZE", "FETCH_SIZE", fetch)
    pmc(out, "pmc_loop1_WRITE_SIZE", "WRITE_SIZE", write_seq)
    r = profsum.loop_bytes(out, "loop1", cal, L=L)
    per = lambda f: k * (f * 1024 * 2 + 0.5 * 1024)
    assert r["dispatches_per_loop"] == k
    assert r["resident_loop_bytes"] == [int(per(100.0))] + [int(per(3.0))] * (L - 1)
    assert r["evict_each_loop_bytes"] == [int(per(100.0))] * L


def test_plain_step_times_are_read_beside_the_traces(tmp_path):
    out = str(tmp_path)
    with open(os.path.join(out, "plain_main.json"), "w") as f:
        f.write("noise\n" + json.dumps(dict(leg="decode_int4_g128_M1", us_per_call=3.92)) + "\n")
    with open(os.path.join(out, "plain_floor.json"), "w") as f:
        f.write(json.dumps(dict(workgroups=768, threads=512, us_per_launch=1.54)) + "\n")
    assert profsum.plain_step_us(out, "main") == 3.92
    assert profsum.plain_step_us(out, "floor") == 1.54
    assert profsum.plain_step_us(out, "gemm") is None
    assert "3.92 us" in profsum.plain_note(3.92, 4.1, "main")
    assert profsum.plain_note(None, 4.1, "main") == ""


def test_valu_counters_per_wave(tmp_path):
    out = str(tmp_path)
    vals = dict(SQ_WAVES=6144.0, SQ_INSTS_VALU=6144.0 * 130, SQ_INSTS_VMEM_RD=6144.0 * 4, SQ_INSTS_LDS=6144.0 * 20,
                SQ_WAIT_ANY=400.0, SQ_WAIT_INST_ANY=100.0, SQ_WAVE_CYCLES=1000.0)
    for run in ("pmc_main_valu", "pmc_int2_valu"):
        rows, d = [], 0
        for c, v in vals.items():   # a non-GEMV dispatch, then three GEMV ones (the middle one doubled)
            for j, (k, f) in enumerate(((PACK, 9.0), (GEMV, 1.0), (GEMV, 2.0), (GEMV, 1.0))):
                rows.append(dict(Dispatch_Id=j + 1, Kernel_Name=k, Counter_Name=c, Counter_Value=v * f))
        write(os.path.join(out, run, "host", "1", f"{run}_counter_collection.csv"), PMC_COLS, rows)
    v = profsum.valu_counters(out, "pmc_main_valu", "gemv")
    assert v["dispatches"] == 3
    assert v["per_wave"]["SQ_INSTS_VALU"] == 130.0 and v["per_wave"]["SQ_INSTS_VMEM_RD"] == 4.0
    assert v["wait_share"] == 0.4 and v["issue_wait_share"] == 0.1
    md = profsum.valu_file(out, "0" * 16)
    # VALU per chunk: 130 per wave x 6144 waves x 64 lanes over 6144 * 2048 / 32 chunks of 32 INT4 codes
    assert "| 130.0 | 130.0 |" in md
