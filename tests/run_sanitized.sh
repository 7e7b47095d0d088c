#!/bin/bash
# The CPU test suite against sanitizer builds of the library's host code (plan
# construction, CSR validation, argument checks) and of the oracle, both with
# clang's AddressSanitizer and UndefinedBehaviorSanitizer, in one process with
# the sanitizer runtime preloaded. Any report aborts the run.
#
#   bash tests/run_sanitized.sh [pytest args]
set -euo pipefail
cd "$(dirname "$0")/.."
python -m sparse_graph_attention_csr_amd.build --sanitize
python -c "import oracle; oracle.build(sanitize=True)"
rt=$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)
export SGAT_LIBRARY=$PWD/_build/san/libsgattn_san.so
export SGAT_ORACLE_LIBRARY=$PWD/oracle/liboracle_san.so
export ASAN_OPTIONS=detect_leaks=0:halt_on_error=1:abort_on_error=1
export UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1
LD_PRELOAD=$rt python -m pytest tests -m "not gpu" -x -q -p no:cacheprovider "$@"
