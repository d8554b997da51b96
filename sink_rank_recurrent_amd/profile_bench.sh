#!/bin/bash
# Kernel trace and HBM byte counters of bench.py on one MI355X (gfx950).
#
#   sink_rank_recurrent_amd/profile_bench.sh OUT_DIR [bench.py arguments]
#
# 1. rocprofv3 --kernel-trace --stats of `bench.py ARGS --no-cpu` -> OUT_DIR/
#    kernel_trace.md, with the average of the reported form's step kernel
#    (lazy decay) over the headline's timed launches, which follow its
#    pre-roll and settle steps.  The CPU oracle leg launches no kernel; it is
#    left out so that no oracle process runs under the profiler.
# 2. Two --pmc passes over the same headline (FETCH_SIZE, then WRITE_SIZE,
#    counted on the step kernel only; the other forms, workloads and the
#    dense baseline are skipped, which leaves the headline's step launches as
#    they are) and the same two counters on a plain 1 GiB device copy ->
#    OUT_DIR/traffic.json: HBM bytes per timed launch beside the algorithmic
#    bytes of the same run.
# Raw profiler output stays in a temporary directory under /tmp.
set -eu -o pipefail
if [ $# -lt 1 ]; then
  echo "usage: $0 OUT_DIR [bench.py arguments]" >&2
  exit 2
fi
out=$1
shift
root=$(cd "$(dirname "$0")/.." && pwd)
cd "$root"
mkdir -p "$out"
export TMPDIR=/tmp
work=$(mktemp -d /tmp/seedprof.XXXXXX)

find_csv() {
  local f
  for f in $(find "$1" -name "*$2"); do
    echo "$f"
    return 0
  done
  echo "no *$2 under $1" >&2
  return 1
}

json_field() {
  python3 -c "import json,sys
for t in open(sys.argv[1]).read().splitlines():
    if t.startswith('{'): d = json.loads(t)
print(eval(sys.argv[2], {}, {'d': d}))" "$1" "$2"
}

args="$*"
echo "[profile] kernel trace: bench.py $args --no-cpu" >&2
timeout -k 10 900 rocprofv3 --kernel-trace --stats -d "$work/trace" -o trace --output-format csv \
  -- python3 bench.py "$@" --no-cpu > "$out/trace_bench.json" 2> "$out/trace_bench.err"
L=$(json_field "$out/trace_bench.json" "d['config']['layers']")
warm=$(json_field "$out/trace_bench.json" "d['warmup']")
steps=$(json_field "$out/trace_bench.json" "d['steps']")
name=$(json_field "$out/trace_bench.json" "d['config']['workload']")
pre=$(json_field "$out/trace_bench.json" "d['breakdown']['pre_roll_steps']")
python3 -m sink_rank_recurrent_amd.profile_summary trace \
  "$(find_csv "$work/trace" kernel_stats.csv)" "$(find_csv "$work/trace" kernel_trace.csv)" \
  --command "sink_rank_recurrent_amd/profile_bench.sh $out $args   # runs: rocprofv3 --kernel-trace --stats -d <tmp> -o trace --output-format csv -- python3 bench.py $args --no-cpu" \
  --title "Kernel trace: bench.py $args (workload $name, CPU leg left out)" \
  --window "$(((pre + warm) * L)):$((steps * L))" --group "seed_step_kernel (lazy decay)" \
  --out "$out/kernel_trace.md" > "$out/kernel_trace.json"

pmc_args="$args --no-cpu --no-sub --no-variant --no-dense"
for c in FETCH_SIZE WRITE_SIZE; do
  echo "[profile] $c on seed_step_kernel: bench.py $pmc_args" >&2
  timeout -s KILL 900 rocprofv3 --pmc "$c" --kernel-include-regex seed_step_kernel \
    -d "$work/$c" -o "$c" --output-format csv \
    -- python3 bench.py "$@" --no-cpu --no-sub --no-variant --no-dense \
    > "$out/${c}_bench.json" 2> "$out/${c}_bench.err"
  echo "[profile] $c on a plain 1 GiB device copy" >&2
  timeout -s KILL 120 rocprofv3 --pmc "$c" -d "$work/copy_$c" -o "copy_$c" --output-format csv \
    -- python3 bench.py --copy-probe > "$out/copy_${c}.json" 2> "$out/copy_${c}.err"
done
python3 -m sink_rank_recurrent_amd.profile_summary counters \
  --fetch "$(find_csv "$work/FETCH_SIZE" counter_collection.csv)" \
  --write "$(find_csv "$work/WRITE_SIZE" counter_collection.csv)" \
  --copy-fetch "$(find_csv "$work/copy_FETCH_SIZE" counter_collection.csv)" \
  --copy-write "$(find_csv "$work/copy_WRITE_SIZE" counter_collection.csv)" \
  --bench-json "$out/FETCH_SIZE_bench.json" \
  --source sink_rank_recurrent_amd/csrc/seed_step.hip \
  --commands "sink_rank_recurrent_amd/profile_bench.sh $out $args   # runs, for C in FETCH_SIZE WRITE_SIZE: rocprofv3 --pmc C --kernel-include-regex seed_step_kernel -d <tmp> -o C --output-format csv -- python3 bench.py $pmc_args; rocprofv3 --pmc C -d <tmp> -o copy_C --output-format csv -- python3 bench.py --copy-probe" \
  --out "$out/traffic.json" > /dev/null
rm -rf "$work"
echo "[profile] done: $out/kernel_trace.md $out/traffic.json" >&2
