#!/bin/bash
# rocprofv3 passes over one bench layer, then the committed table step:
#   kernel trace + stats, FETCH_SIZE, WRITE_SIZE, SQ/GRBM counters, and the
#   two byte counters over a 1 GiB device copy for their scale.
# Usage: profile_layer.sh CONFIG OUTDIR   (CONFIG: c2, c3, c4, c5; run on a GPU
# host from anywhere; writes OUTDIR/CONFIG/... and profiles/layer_kernels_*).
# CONFIG gather: the isolated column gather on the 128K layer's inputs
# (bench.py --gather-only; trace, FETCH_SIZE and WRITE_SIZE passes) ->
# profiles/gather_vs_llama8b_128k_bf16.*
# Each pass runs under its own time limit and the script stops at the first
# failure.  With PROFILE_TABLES_ONLY=1 it only rebuilds the tables from the
# CSV files already in OUTDIR (no GPU needed).
set -u
C=$1
O=$(realpath -m "$2")
R=$(cd "$(dirname "$0")/.." && pwd)
B="--no-cpu-baseline --no-1m --no-dense --no-exact --no-gather --no-antidiag"
T=${PROFILE_PASS_SECONDS:-400}
mkdir -p "$O/$C"
cd /tmp && export TMPDIR=/tmp
step() { echo "[profile_layer] $C: $1"; }
if [ "$C" = gather ]; then
  G="--config c3 --gather-only"
  if [ "${PROFILE_TABLES_ONLY:-0}" != 1 ]; then
    if [ ! -d "$O/copy_fetch" ] || [ ! -d "$O/copy_write" ]; then
      step "copy calibration"
      timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE -d "$O/copy_fetch" -o pmc --output-format csv -- python3 "$R/bench.py" --calibrate-copy > "$O/copy_fetch.log" 2>&1 || exit $?
      timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE -d "$O/copy_write" -o pmc --output-format csv -- python3 "$R/bench.py" --calibrate-copy > "$O/copy_write.log" 2>&1 || exit $?
    fi
    step "trace"
    timeout -k 10 "$T" rocprofv3 --kernel-trace --stats -d "$O/$C/trace" -o trace --output-format csv -- python3 "$R/bench.py" $G > "$O/$C.trace.log" 2>&1 || exit $?
    step "FETCH_SIZE"
    timeout -s KILL "$T" rocprofv3 --pmc FETCH_SIZE -d "$O/$C/fetch" -o pmc --output-format csv -- python3 "$R/bench.py" $G > "$O/$C.fetch.log" 2>&1 || exit $?
    step "WRITE_SIZE"
    timeout -s KILL "$T" rocprofv3 --pmc WRITE_SIZE -d "$O/$C/write" -o pmc --output-format csv -- python3 "$R/bench.py" $G > "$O/$C.write.log" 2>&1 || exit $?
  fi
  step "tables"
  cd "$R" && python3 -m dynamic_sparse_attention_amd.profile_tables --gather --workload c3 --steps 8 \
    --trace "$O/$C/trace" --fetch "$O/$C/fetch" --write "$O/$C/write" \
    --copy-fetch "$O/copy_fetch" --copy-write "$O/copy_write" --bench-log "$O/$C.trace.log" \
    --command "dynamic_sparse_attention_amd/profile_layer.sh gather OUT   # from the repository root; the passes it runs:
rocprofv3 --kernel-trace --stats -d OUT/gather/trace -o trace --output-format csv -- python3 bench.py $G
rocprofv3 --pmc FETCH_SIZE -d OUT/gather/fetch -o pmc --output-format csv -- python3 bench.py $G
rocprofv3 --pmc WRITE_SIZE -d OUT/gather/write -o pmc --output-format csv -- python3 bench.py $G
rocprofv3 --pmc FETCH_SIZE -d OUT/copy_fetch -o pmc --output-format csv -- python3 bench.py --calibrate-copy
rocprofv3 --pmc WRITE_SIZE -d OUT/copy_write -o pmc --output-format csv -- python3 bench.py --calibrate-copy
python3 -m dynamic_sparse_attention_amd.profile_tables --gather --workload c3 --steps 8 --trace OUT/gather/trace --fetch OUT/gather/fetch --write OUT/gather/write --copy-fetch OUT/copy_fetch --copy-write OUT/copy_write --bench-log OUT/gather.trace.log" || exit $?
  step "done"
  exit 0
fi
if [ "${PROFILE_TABLES_ONLY:-0}" = 1 ]; then
  :
else
if [ ! -d "$O/copy_fetch" ] || [ ! -d "$O/copy_write" ]; then
  step "copy calibration"
  timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE -d "$O/copy_fetch" -o pmc --output-format csv -- python3 "$R/bench.py" --calibrate-copy > "$O/copy_fetch.log" 2>&1 || exit $?
  timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE -d "$O/copy_write" -o pmc --output-format csv -- python3 "$R/bench.py" --calibrate-copy > "$O/copy_write.log" 2>&1 || exit $?
fi
step "trace"
timeout -k 10 "$T" rocprofv3 --kernel-trace --stats -d "$O/$C/trace" -o trace --output-format csv -- python3 "$R/bench.py" --config "$C" $B --steps 2 --warmup 1 > "$O/$C.trace.log" 2>&1 || exit $?
step "FETCH_SIZE"
timeout -s KILL "$T" rocprofv3 --pmc FETCH_SIZE -d "$O/$C/fetch" -o pmc --output-format csv -- python3 "$R/bench.py" --config "$C" $B --steps 1 --warmup 0 > "$O/$C.fetch.log" 2>&1 || exit $?
step "WRITE_SIZE"
timeout -s KILL "$T" rocprofv3 --pmc WRITE_SIZE -d "$O/$C/write" -o pmc --output-format csv -- python3 "$R/bench.py" --config "$C" $B --steps 1 --warmup 0 > "$O/$C.write.log" 2>&1 || exit $?
step "SQ counters"
timeout -s KILL "$T" rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAVES -d "$O/$C/sq" -o pmc --output-format csv -- python3 "$R/bench.py" --config "$C" $B --steps 1 --warmup 0 > "$O/$C.sq.log" 2>&1 || exit $?
fi
step "tables"
cd "$R" && python3 -m dynamic_sparse_attention_amd.profile_tables --workload "$C" --steps 3 \
  --trace "$O/$C/trace" --fetch "$O/$C/fetch" --write "$O/$C/write" --sq "$O/$C/sq" \
  --copy-fetch "$O/copy_fetch" --copy-write "$O/copy_write" --bench-log "$O/$C.trace.log" \
  --command "dynamic_sparse_attention_amd/profile_layer.sh $C OUT   # from the repository root; the passes it runs:
rocprofv3 --kernel-trace --stats -d OUT/$C/trace -o trace --output-format csv -- python3 bench.py --config $C $B --steps 2 --warmup 1
rocprofv3 --pmc FETCH_SIZE -d OUT/$C/fetch -o pmc --output-format csv -- python3 bench.py --config $C $B --steps 1 --warmup 0
rocprofv3 --pmc WRITE_SIZE -d OUT/$C/write -o pmc --output-format csv -- python3 bench.py --config $C $B --steps 1 --warmup 0
rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAVES -d OUT/$C/sq -o pmc --output-format csv -- python3 bench.py --config $C $B --steps 1 --warmup 0
rocprofv3 --pmc FETCH_SIZE -d OUT/copy_fetch -o pmc --output-format csv -- python3 bench.py --calibrate-copy
rocprofv3 --pmc WRITE_SIZE -d OUT/copy_write -o pmc --output-format csv -- python3 bench.py --calibrate-copy
python3 -m dynamic_sparse_attention_amd.profile_tables --workload $C --steps 3 --trace OUT/$C/trace --fetch OUT/$C/fetch --write OUT/$C/write --sq OUT/$C/sq --copy-fetch OUT/copy_fetch --copy-write OUT/copy_write --bench-log OUT/$C.trace.log" || exit $?
step "done"
