#!/bin/bash
# Collect, for each bench.py workload named, a rocprofv3 kernel trace with
# per-kernel statistics and four counter passes (FETCH_SIZE; WRITE_SIZE;
# matrix-core busy cycles and bf16 MFMA operations, LDS bank conflicts and LDS
# activity, GPU active cycles; instruction counts and VALU / matrix-core issue
# overlap), plus FETCH_SIZE and WRITE_SIZE for a plain
# 1 GiB device copy (calibration).  A workload may carry a forced split count
# as NAME:sN (e.g. long_ctx:s64); its files are tagged NAME_sN.
# usage: bash paged_kv_split_amd/profiling/collect.sh OUTDIR WORKLOAD...
set -u
cd "$(dirname "$0")/../.." || exit 1
export TMPDIR=/tmp
out=$1
shift
mkdir -p "$out"
# the kernel trace times each workload as bench.py does by default (20
# warmup calls, then timed runs of 200); the counter passes need only a few
# calls each
BENCH="python3 -u bench.py --no-cpu-baseline --no-configs"
TRACE="--warmup 20 --steps 200 --runs 2"
COUNT="--warmup 3 --steps 4 --runs 1"

step() {  # step TAG LIMIT_SECONDS COMMAND...
  local tag=$1 lim=$2
  shift 2
  echo "step $tag" >&2
  timeout -s KILL "$lim" "$@" > "$out/$tag.out" 2> "$out/$tag.log"
  local rc=$?
  if [ $rc -ne 0 ]; then
    echo "failed: $tag (status $rc)" >&2
    tail -5 "$out/$tag.log" >&2
    exit $rc
  fi
}

step copy_fetch 120 rocprofv3 --pmc FETCH_SIZE -d "$out/copy_fetch" -o copy_fetch --output-format csv -- \
  python3 -u bench.py --copy-calibration 1073741824
step copy_write 120 rocprofv3 --pmc WRITE_SIZE -d "$out/copy_write" -o copy_write --output-format csv -- \
  python3 -u bench.py --copy-calibration 1073741824
for key in "$@"; do
  wl=${key%%:*}
  extra=""
  tag=$wl
  if [ "$key" != "$wl" ]; then
    extra="--splits ${key##*:s}"
    tag="${wl}_s${key##*:s}"
  fi
  BW="$BENCH $extra"
  wl=$tag
  name=${key%%:*}
  step "${wl}_trace" 300 rocprofv3 --kernel-trace --stats -d "$out/${wl}_trace" -o trace --output-format csv -- \
    $BW --workload "$name" $TRACE
  step "${wl}_fetch" 120 rocprofv3 --pmc FETCH_SIZE -d "$out/${wl}_fetch" -o fetch --output-format csv -- \
    $BW --workload "$name" $COUNT
  step "${wl}_write" 120 rocprofv3 --pmc WRITE_SIZE -d "$out/${wl}_write" -o write --output-format csv -- \
    $BW --workload "$name" $COUNT
  step "${wl}_sq" 120 rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_LDS_BANK_CONFLICT \
    SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE MfmaUtil -d "$out/${wl}_sq" -o sq --output-format csv -- \
    $BW --workload "$name" $COUNT
  step "${wl}_issue" 120 rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_VALU_TRANS_F32 \
    SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_COEXEC_CYCLES SQ_WAVES SQ_WAVE_CYCLES GRBM_GUI_ACTIVE \
    -d "$out/${wl}_issue" -o issue --output-format csv -- $BW --workload "$name" $COUNT
done
echo "collected in $out" >&2
