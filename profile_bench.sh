#!/bin/bash
# Profile one bench.py workload under rocprofv3 on one MI355X: a kernel trace
# and three counter passes (FETCH_SIZE; WRITE_SIZE; clock + MFMA busy), each a
# run of its own over the same bench command, then nothing else. The databases
# and the launch table land in gpurun_out/prof_<workload>/; turn them into the
# profiles/ summaries with
#   python3 bench.py --summarize gpurun_out/prof_<workload> --workload <workload>
#
# usage: bash profile_bench.sh WORKLOAD [STEPS]
set -o pipefail
W=${1:?usage: profile_bench.sh WORKLOAD [STEPS]}
S=${2:-3}
D=gpurun_out/prof_$W
rm -rf "$D"
mkdir -p "$D"
export TMPDIR=/tmp
BENCH="python3 -u bench.py --workload $W --steps $S --warmup 1 --no-cpu-baseline --record $D/items.json"
echo "cd /root/repo && export TMPDIR=/tmp   # then:" > "$D/commands.txt"

pass() {   # pass NAME ROCPROF-OPTIONS...
    local name=$1
    shift
    local cmd="timeout -s KILL 300 rocprofv3 $* -d $D -o $name -- $BENCH"
    echo "$cmd" >> "$D/commands.txt"
    echo "[profile_bench] $W: pass $name" >&2
    $cmd > "$D/$name.log" 2>&1
    local rc=$?
    tail -3 "$D/$name.log" >&2
    # the profiler itself may end with a segmentation fault after the program
    # has finished and its results are whole: accept that when the bench line
    # was printed
    if [ $rc -eq 139 ] && grep -q '^{"metric"' "$D/$name.log"; then
        echo "[profile_bench] $W: pass $name: profiler exited 139 after a complete run" >&2
        rc=0
    fi
    if [ $rc -ne 0 ]; then
        echo "[profile_bench] $W: pass $name exited with $rc" >&2
        exit $rc
    fi
}

pass trace --kernel-trace --stats
pass fetch --pmc FETCH_SIZE
pass write --pmc WRITE_SIZE
pass util --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES
echo "[profile_bench] $W: done" >&2
