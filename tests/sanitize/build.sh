#!/bin/bash
# Builds tests/sanitize/_build/host_check: the C ABI layer's host code and the
# CPU oracle with AddressSanitizer and UndefinedBehaviorSanitizer (host code
# only; the gfx950 device code of the library is built as usual and never
# runs), linked with the library's other objects. Needs the objects of a
# library build (dsa_top_token_amd/_build).
set -euo pipefail
ROOT="$(cd "$(dirname "$0")/../.." && pwd)"
OUT="$ROOT/tests/sanitize/_build"
mkdir -p "$OUT"
HIPCC=/opt/rocm/bin/hipcc
CLANG=/opt/rocm/lib/llvm/bin/clang
SAN="-fsanitize=address,undefined -fno-sanitize-recover=all -fno-omit-frame-pointer"
$HIPCC --offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -I"$ROOT/include" \
    -Xclang -target-feature -Xclang -packed-fp32-ops \
    -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
    -Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer \
    -x hip -c "$ROOT/dsa_top_token_amd/csrc/api.cpp" -o "$OUT/api.o"
$CLANG -O1 -g -std=c11 $SAN -c "$ROOT/oracle/dsa_oracle.c" -o "$OUT/oracle.o"
$CLANG -O1 -g -std=c11 $SAN -c "$ROOT/tests/sanitize/host_check.c" -o "$OUT/host_check.o"
OBJS=""
for s in indexer.hip topk.hip decode.hip prefill.hip attn.hip threshold.hip project.hip; do
    OBJS="$OBJS $ROOT/dsa_top_token_amd/_build/$s.o"
done
$HIPCC --offload-arch=gfx950 -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
    "$OUT/host_check.o" "$OUT/oracle.o" "$OUT/api.o" $OBJS -o "$OUT/host_check" -lm
echo "$OUT/host_check"
