#!/bin/bash
# Profiles the benchmark legs with rocprofv3 on one GPU: kernel traces
# (per-dispatch durations) and the HBM byte counters FETCH_SIZE / WRITE_SIZE,
# each counter in a run of its own, plus the plain copy that calibrates them.
#
#   bash bit_weight_only_dequant_amd/profile.sh OUTDIR
#   python3 -m bit_weight_only_dequant_amd.profsum OUTDIR --write profiles
#
# With a second argument `valu` only the instruction-count passes of the M = 1
# GEMVs run (summarised by profsum ... --part valu).
#
# Every step runs under its own time limit and the script stops at the first
# failure.
set -eo pipefail
R=$(cd "$(dirname "${BASH_SOURCE[0]}")/.." && pwd)
mkdir -p "$1"
OUT=$(cd "$1" && pwd)
cd /tmp
export TMPDIR=/tmp

step() {   # step NAME LIMIT_S ROCPROF_ARGS... -- BENCH_ARGS...
  local name=$1 limit=$2
  shift 2
  local prof=()
  while [ "$1" != "--" ]; do prof+=("$1"); shift; done
  shift
  echo "== $name: rocprofv3 ${prof[*]} -- python3 bench.py $*"
  timeout -k 10 -s KILL "$limit" rocprofv3 "${prof[@]}" --output-format csv -d "$OUT/$name" -o "$name" \
    -- python3 "$R/bench.py" "$@" > "$OUT/$name.log" 2>&1
  echo "   done"
}

# first import of torch on a fresh machine pages the image in: not profiled
timeout -k 10 300 python3 -c "import torch; print(torch.__version__)"

# instructions issued and cycles waited per wave by the M = 1 GEMVs (INT4
# decode shape; INT2 g64, N = 8192): seven SQ counters, one pass each
VALU_COUNTERS=(SQ_WAVES SQ_INSTS_VALU SQ_INSTS_VMEM_RD SQ_INSTS_LDS SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAVE_CYCLES)
step pmc_main_valu 180 --pmc "${VALU_COUNTERS[@]}" -- --only main --steps 81 --warmup 8
step pmc_int2_valu 180 --pmc "${VALU_COUNTERS[@]}" -- --only int2 --steps 103 --warmup 8
if [ "$2" = "valu" ]; then
  echo "profile runs complete: $OUT"
  exit 0
fi

# the traced legs once without the profiler, on this machine: the step times
# the traced durations are read against
for leg in main gemm floor; do
  echo "== plain_$leg: python3 bench.py --only $leg"
  timeout -k 10 300 python3 "$R/bench.py" --only "$leg" > "$OUT/plain_$leg.json" 2> "$OUT/plain_$leg.log"
  echo "   done"
done

step trace_main 300 --kernel-trace --stats -- --only main
step trace_gemm 300 --kernel-trace --stats -- --only gemm
step trace_stream 300 --kernel-trace --stats -- --only stream
step trace_floor 300 --kernel-trace --stats -- --only floor
step trace_loop128 300 --kernel-trace --stats -- --only loop --loop-m 128
step trace_loop1 300 --kernel-trace --stats -- --only loop --loop-m 1
step pmc_gemm_mfma 180 --pmc SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE \
  -- --only gemm --steps 64 --warmup 8
for c in FETCH_SIZE WRITE_SIZE; do
  step "pmc_copy_$c" 120 --pmc "$c" -- --only copy
  step "pmc_main_$c" 180 --pmc "$c" -- --only main --steps 81 --warmup 8
  step "pmc_gemm_$c" 180 --pmc "$c" -- --only gemm --steps 64 --warmup 8
  step "pmc_loop128_$c" 180 --pmc "$c" -- --only loop_prof --loop-m 128
  step "pmc_loop1_$c" 180 --pmc "$c" -- --only loop_prof --loop-m 1
done
for m in 128 1; do   # L2-miss latency: in-flight reads accumulated per cycle, and their count
  step "pmc_loop${m}_lat" 180 --pmc TCC_EA0_RDREQ_LEVEL_sum TCC_EA0_RDREQ_sum -- --only loop_prof --loop-m "$m"
done
# the M = 1 block in one persistent launch: L = 1 against L = 8
for c in FETCH_SIZE WRITE_SIZE; do
  step "pmc_persist_$c" 180 --pmc "$c" -- --only loop_prof_persistent
done
step pmc_persist_lat 180 --pmc TCC_EA0_RDREQ_LEVEL_sum TCC_EA0_RDREQ_sum -- --only loop_prof_persistent
echo "profile runs complete: $OUT"
