#!/bin/bash
# Instruction and cycle counters of the compression kernel on one MI355X.
#
#   sink_rank_recurrent_amd/profile_compress.sh OUT_DIR [CASE ...]
#
# Two rocprofv3 --pmc passes (at most 8 SQ counters each) over each of:
#   n48: one layer of workload 5 (256 requests x 32 GDN heads, 8192 units,
#        R = 16, W = 32: every compression of n = 48 columns);
#   n80: workload 4 (64 requests x 32 KDA heads, 2048 units, R = 16, W = 64:
#        n = 80, two waves per unit),
# counted on the fp32 compression instance only, and
#   conv: the end-of-prefill conversion of workload 2 (1024 dense 128 x 128
#        states to rank 16, two waves per unit, the conversion instance),
# then summarised per dispatch and per wave ->
# OUT_DIR/counters_compress_wave_<case>.md.  CASE limits the run to the
# cases named (default: all three).
# Raw profiler output stays in a temporary directory under /tmp.
set -eu -o pipefail
if [ $# -lt 1 ]; then
  echo "usage: $0 OUT_DIR [n48|n80|conv ...]" >&2
  exit 2
fi
out=$1
shift
cases=${*:-n48 n80 conv}
for case in $cases; do
  case $case in
    n48|n80|conv) ;;
    *) echo "unknown case $case (n48, n80 or conv)" >&2; exit 2 ;;
  esac
done
root=$(cd "$(dirname "$0")/.." && pwd)
cd "$root"
mkdir -p "$out"
export TMPDIR=/tmp
work=$(mktemp -d /tmp/seedcprof.XXXXXX)
p1="SQ_WAVES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_INSTS_MFMA SQ_WAVE_CYCLES SQ_BUSY_CYCLES"
p2="SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_LDS_BANK_CONFLICT"
for case in $cases; do
  regex='compress_wave_kernel<[0-9]+, [0-9]+, [0-9]+, [0-9]+, 0>'
  if [ "$case" = conv ]; then
    args="--workload 2 --no-cpu --no-dense --no-variant --no-sub --steps 32 --warmup 0"
    units=1024
    wpu=2
    regex='compress_wave_kernel<128, 16, 128, 128, 4>'
  elif [ "$case" = n48 ]; then
    args="--workload 5 --layers 1 --no-cpu --no-dense --no-variant --no-sub --steps 64 --warmup 0"
    units=8192
    wpu=1
  else
    args="--workload 4 --no-cpu --no-dense --no-variant --no-sub --steps 128 --warmup 0"
    units=2048
    wpu=2
  fi
  csvs=""
  for pass in 1 2; do
    if [ $pass = 1 ]; then ctr=$p1; else ctr=$p2; fi
    echo "[profile] $case pass $pass: $ctr" >&2
    timeout -k 10 600 rocprofv3 --pmc $ctr --kernel-include-regex "$regex" \
      -d "$work/${case}_$pass" -o "p$pass" --output-format csv \
      -- python3 bench.py $args > "$out/${case}_p$pass.json" 2> "$out/${case}_p$pass.err"
    csvs="$csvs $(find "$work/${case}_$pass" -name '*counter_collection.csv' -print -quit)"
  done
  python3 -m sink_rank_recurrent_amd.profile_summary pmc $csvs --kernel "$regex" --units $units --waves-per-unit $wpu \
    --title "Counters of the compression kernel ($case): bench.py $args" \
    --command "sink_rank_recurrent_amd/profile_compress.sh $out $case   # runs, for the two counter sets: rocprofv3 --pmc <set> --kernel-include-regex '$regex' -d <tmp> -o p<k> --output-format csv -- python3 bench.py $args; set 1: $p1; set 2: $p2" \
    --out "$out/counters_compress_wave_$case.md" > /dev/null
done
rm -rf "$work"
echo "[profile] done: $(for c in $cases; do printf "%s " "$out/counters_compress_wave_$c.md"; done)" >&2
