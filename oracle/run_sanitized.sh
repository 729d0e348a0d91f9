#!/bin/bash
# Run the oracle's CPU tests (-m "not gpu") against a copy of the oracle built
# with AddressSanitizer and UndefinedBehaviorSanitizer (host code only: the
# oracle is plain C).  The instrumented library replaces oracle/libtkv_oracle.so
# for the run; a normal build is restored afterwards.
set -euo pipefail
cd "$(dirname "$0")/.."
LIB=oracle/libtkv_oracle.so
gcc -O1 -g -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -fPIC -shared \
    -fsanitize=address,undefined -fno-sanitize-recover=undefined -fno-omit-frame-pointer \
    -o "$LIB" oracle/tkv_oracle.c -lm
status=0
ASAN_OPTIONS=detect_leaks=0:abort_on_error=1 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
LD_PRELOAD="$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so)" \
    python3 -m pytest tests -m "not gpu" -x -q -p no:cacheprovider "$@" || status=$?
python3 -c "import oracle; oracle.build(force=True)"
exit $status
