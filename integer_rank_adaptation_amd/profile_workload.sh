#!/bin/bash
# rocprofv3 passes over a few steps of one benchmark workload, then the per-kernel
# summaries (profiles/).  Usage, from the repository root, on one MI355X:
#
#   bash integer_rank_adaptation_amd/profile_workload.sh WORKLOAD OUTDIR [bench options...]
#
# Passes (each a run of its own; counters are never combined with tracing):
#   trace    --kernel-trace --stats                 kernel durations
#   fetch    --pmc FETCH_SIZE                       HBM read bytes (calibrated below)
#   write    --pmc WRITE_SIZE                       HBM write bytes
#   sq       --pmc 8 SQ counters + GRBM_GUI_ACTIVE  VALU / MFMA / LDS activity, clock
#   derived  --pmc MfmaUtil VALUBusy                rocprofv3's derived busy percentages
#   copy_*   FETCH_SIZE / WRITE_SIZE of a plain 1 GiB device copy (the calibration)
# Every pass runs under its own time limit and the script stops at the first failure.
# PASSES (environment, default "trace fetch write sq derived copy") selects passes.
set -euo pipefail
WL=${1:?workload index}
OUT=${2:?output directory}
shift 2
ROOT=$(cd "$(dirname "$0")/.." && pwd)
mkdir -p "$OUT"
OUT=$(cd "$OUT" && pwd)
BENCH=(python3 "$ROOT/bench.py" --workload "$WL" --steps 10 --warmup 3 --no-cpu-baseline --no-ptq --no-fused
       --no-codes --no-ste --no-graph --no-overlap --no-aux-laws --no-sweep --no-grouped --no-library-gemm
       --kernel-runs 0 "$@")
cd /tmp
export TMPDIR=/tmp
run() {
  local name=$1
  shift
  echo "[profile] $name" >&2
  timeout -s KILL 240 rocprofv3 "$@" --output-format csv -d "$OUT/$name" -o "$name" -- "${BENCH[@]}" \
    > "$OUT/$name.log" 2>&1
}
PASSES=${PASSES:-"trace fetch write sq derived copy"}
want() { [[ " $PASSES " == *" $1 "* ]]; }
if want trace; then run trace --kernel-trace --stats; fi
if want fetch; then run fetch --pmc FETCH_SIZE; fi
if want write; then run write --pmc WRITE_SIZE; fi
if want sq; then
  run sq --pmc SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_I8 SQ_WAVES \
    SQ_BUSY_CU_CYCLES SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE
fi
if want derived; then run derived --pmc MfmaUtil VALUBusy; fi
if want copy; then
  for c in FETCH_SIZE WRITE_SIZE; do
    echo "[profile] copy $c" >&2
    timeout -s KILL 120 rocprofv3 --pmc "$c" --output-format csv -d "$OUT/copy_$c" -o "copy_$c" -- \
      python3 "$ROOT/bench.py" --copy-probe 1024 > "$OUT/copy_$c.log" 2>&1
  done
fi
echo "[profile] done" >&2
