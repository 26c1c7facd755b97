#!/bin/bash
# The CPU test suite (pytest -m "not gpu") with AddressSanitizer and
# UndefinedBehaviorSanitizer in the host code it runs: the oracle library and the
# library's host translation units (the C ABI and the step cache), linked with
# the ordinary device-code objects.  No GPU is needed or used.
#   bash tests/run_host_sanitizers.sh [extra pytest arguments]
set -euo pipefail
REPO="$(cd "$(dirname "$0")/.." && pwd)"
OUT="$REPO/embedding_table_gather_amd/_build/sanitize"
mkdir -p "$OUT"
LLVM=/opt/rocm/llvm
SAN="-fsanitize=address,undefined -fno-sanitize-recover=undefined -fno-omit-frame-pointer -g"

# the ordinary objects (device code of every .hip source)
python3 "$REPO/embedding_table_gather_amd/build.py"

# oracle: same flags as its normal build, OpenMP left out (the loops run serially)
"$LLVM/bin/clang" -O1 -std=c11 -ffp-contract=off -fno-fast-math $SAN -shared -fPIC \
  -o "$OUT/liboracle_san.so" "$REPO/oracle/etg_oracle.c" -lm

# host translation units with the sanitizers; the rest as built above
CSRC="$REPO/embedding_table_gather_amd/csrc"
for f in etg_api step; do
  /opt/rocm/bin/hipcc -O1 -fPIC -std=c++17 -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
    -Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer -g \
    -c "$CSRC/$f.cpp" -o "$OUT/$f.o"
done
objs=""
for f in gather logits stream wide gemm rank q8 row probe noalloc; do objs="$objs $REPO/embedding_table_gather_amd/_build/$f.o"; done
/opt/rocm/bin/hipcc --offload-arch=gfx950 -shared -fPIC -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
  -shared-libsan -o "$OUT/libetg_san.so" "$OUT/etg_api.o" "$OUT/step.o" $objs

RT="$("$LLVM/bin/clang" -print-file-name=libclang_rt.asan-x86_64.so)"
cd "$REPO"
# Python and its extension modules are not instrumented: leak reports are off
ETG_LIBRARY="$OUT/libetg_san.so" ETG_ORACLE_LIBRARY="$OUT/liboracle_san.so" LD_PRELOAD="$RT" \
  ASAN_OPTIONS=detect_leaks=0:abort_on_error=1 UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1 \
  python3 -m pytest tests -m "not gpu" -q -p no:cacheprovider "$@"
