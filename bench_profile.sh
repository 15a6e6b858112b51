#!/bin/bash
# Regenerates the rocprofv3 summaries kept under profiles/ (run from the
# repository root on a machine with the GPU; raw output goes to $1).
#
#   bash bench_profile.sh <raw-output-dir> [summaries]
#
# With "summaries" only the text summaries are written again from the raw
# output already in the directory (no GPU needed).
#
# 1. kernel trace + stats of the default bench run (every workload row) and
#    of the headline workload alone;
# 2. FETCH_SIZE then WRITE_SIZE (one counter per run) for the headline
#    workload's kernels, for the same workload run non-causal (the reduction
#    pass and the apply pass), and for the decode kernel, and the same two
#    counters for a plain 256 MiB copy, which calibrates them into bytes;
# 3. one pass of SQ counters over every workload: matrix-core utilisation
#    (MfmaUtil), matrix-core flops, and the waves' wait and LDS shares.
# The summaries are written next to the raw output as *.txt.
set -euo pipefail
OUT=${1:?raw output directory}
mkdir -p "$OUT"
export TMPDIR=${TMPDIR:-/tmp}
SRC="sequence_mixing_amd/csrc/linattn_fmt.hip sequence_mixing_amd/csrc/linattn_kern.h sequence_mixing_amd/csrc/linattn_plan.h sequence_mixing_amd/csrc/linattn_plan.cpp"
KR="k_causal_chunks|k_seg_totals|k_seg_scan|k_noncausal_apply"

step() { echo "== $*"; }

C1="rocprofv3 --kernel-trace --stats -f csv -d $OUT/trace_all -o run -- python3 bench.py --cpu-seconds 2"
C2="rocprofv3 --kernel-trace --stats -f csv -d $OUT/trace_cfg2 -o run -- python3 bench.py --cold-only --cpu-seconds 0"
CTRS="MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS SQ_LDS_BANK_CONFLICT"
C3="rocprofv3 --pmc $CTRS --kernel-include-regex '$KR|k_decode_step|k_bwd' -f csv -d $OUT/counters_all -o run -- python3 bench.py --rows 1 --steps 5 --warmup 2 --cpu-seconds 0"
if [ "${2:-}" != "summaries" ]; then
step "trace: default bench"
timeout -k 10 600 $C1 > "$OUT/trace_all.json" 2> "$OUT/trace_all.err"
step "trace: headline workload"
timeout -k 10 300 $C2 > "$OUT/trace_cfg2.json" 2> "$OUT/trace_cfg2.err"
for ctr in FETCH_SIZE WRITE_SIZE; do
    step "$ctr: headline workload"
    timeout -s KILL 200 rocprofv3 --pmc $ctr --kernel-include-regex "$KR" -f csv -d $OUT/${ctr}_cfg2 -o run -- \
        python3 bench.py --cold-only --steps 5 --warmup 2 --cpu-seconds 0 > "$OUT/${ctr}_cfg2.out" 2>&1
    step "$ctr: headline workload, non-causal"
    timeout -s KILL 200 rocprofv3 --pmc $ctr --kernel-include-regex "$KR" -f csv -d $OUT/${ctr}_nc -o run -- \
        python3 bench.py --causal 0 --cold-only --steps 5 --warmup 2 --cpu-seconds 0 > "$OUT/${ctr}_nc.out" 2>&1
    step "$ctr: decode"
    timeout -s KILL 300 rocprofv3 --pmc $ctr --kernel-include-regex "k_decode_step" -f csv -d $OUT/${ctr}_decode -o run -- \
        python3 bench.py --rows 1 --steps 5 --warmup 2 --cpu-seconds 0 > "$OUT/${ctr}_decode.out" 2>&1
    step "$ctr: copy calibration"
    timeout -s KILL 90 rocprofv3 --pmc $ctr -f csv -d $OUT/${ctr}_copy -o run -- \
        python3 bench_calib_copy.py 256 > "$OUT/${ctr}_copy.out" 2>&1
done

step "counters: every workload"
timeout -s KILL 500 rocprofv3 --pmc $CTRS --kernel-include-regex "$KR|k_decode_step|k_bwd" -f csv -d $OUT/counters_all -o run -- \
    python3 bench.py --rows 1 --steps 5 --warmup 2 --cpu-seconds 0 > "$OUT/counters_all.out" 2>&1
fi

PMC="rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --kernel-include-regex '<kernels>' -f csv -- python3 bench.py --steps 5 --warmup 2 --cpu-seconds 0 (--cold-only headline, --causal 0 --cold-only non-causal, --rows 1 decode); calibration: rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -- python3 bench_calib_copy.py 256"
python3 bench_profsum.py "$OUT/trace_all/run_kernel_stats.csv" "$C1" \
    "all kernels of the default bench run (every workload row; bench JSON in the same run)" > "$OUT/kernels_all_workloads.txt"
python3 bench_profsum.py "$OUT/trace_cfg2/run_kernel_stats.csv" "$C2" \
    "headline workload, cold launches only: causal fp32 B2 H8 N4096 d64 (k_causal_chunks dominant)" > "$OUT/k_causal_chunks_f32_B2H8N4096d64.txt"
python3 bench_profsum.py traffic cfg2 "$OUT/FETCH_SIZE_cfg2/run_counter_collection.csv" \
    "$OUT/WRITE_SIZE_cfg2/run_counter_collection.csv" "$OUT/FETCH_SIZE_copy/run_counter_collection.csv" \
    "$OUT/WRITE_SIZE_copy/run_counter_collection.csv" 256 "$PMC" $SRC > "$OUT/traffic_cfg2_f32_B2H8N4096d64.txt"
python3 bench_profsum.py traffic cfg2_noncausal "$OUT/FETCH_SIZE_nc/run_counter_collection.csv" \
    "$OUT/WRITE_SIZE_nc/run_counter_collection.csv" "$OUT/FETCH_SIZE_copy/run_counter_collection.csv" \
    "$OUT/WRITE_SIZE_copy/run_counter_collection.csv" 256 "$PMC" $SRC > "$OUT/traffic_cfg2_noncausal_f32_B2H8N4096d64.txt"
python3 bench_profsum.py counters "$OUT/counters_all/run_counter_collection.csv" "$C3" \
    "SQ counters per kernel over every workload of the default bench run (matrix-core use, waits, LDS)" \
    > "$OUT/counters_all_workloads.txt"
python3 bench_profsum.py traffic decode "$OUT/FETCH_SIZE_decode/run_counter_collection.csv" \
    "$OUT/WRITE_SIZE_decode/run_counter_collection.csv" "$OUT/FETCH_SIZE_copy/run_counter_collection.csv" \
    "$OUT/WRITE_SIZE_copy/run_counter_collection.csv" 256 "$PMC" $SRC > "$OUT/traffic_decode_bf16_B64H32Hkv8d128.txt"
grep -h "^headline\|^cfg\|^decay\|^packed" "$OUT/trace_all.err" > "$OUT/bench_rows_under_trace.txt" || true
step "done"
