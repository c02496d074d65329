#!/bin/bash
# The CPU test suite (-m "not gpu") with AddressSanitizer and UndefinedBehaviorSanitizer
# on the oracle and on the host side of the HIP library (argument validation, plans,
# workspace layouts): both are rebuilt with the sanitizers, the ROCm toolchain's
# sanitizer runtime is preloaded into the (uninstrumented) Python, and the loaders
# are pointed at the sanitized builds.  A report fails the run.  CPU only.
set -e
ROOT="$(cd "$(dirname "$0")/.." && pwd)"
cd "$ROOT"
python3 oracle/build.py --sanitize
python3 mxfp4_bit_weight_amd/build.py --sanitize
RT="$(/opt/rocm/lib/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so)"
# leaks: CPython keeps its arenas until exit; the allocator's own checks stay on
export ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:allocator_may_return_null=1"
export UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1"
export FP4W_ORACLE_LIB="$ROOT/oracle/liboracle_san.so"
export FP4W_LIB="$ROOT/mxfp4_bit_weight_amd/libfp4w_san.so"
LD_PRELOAD="$RT" python3 -m pytest tests -x -q -m "not gpu" -p no:cacheprovider "$@"
