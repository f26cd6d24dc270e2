#!/bin/bash
# Builds the host-side ABI checks against k2_api.cpp compiled with AddressSanitizer and
# UndefinedBehaviorSanitizer on its host code (device code is built as usual), linked with the other
# library objects of the normal build, and runs them. No GPU is needed: every checked call fails
# validation or only queries sizes before any device work.
# Usage: tests/sanitize/build_and_run.sh OUTDIR   (needs flow_matching_diffusion_amd/_build/*.o)
set -euo pipefail
HERE="$(cd "$(dirname "$0")" && pwd)"
ROOT="$(cd "$HERE/../.." && pwd)"
OUT="${1:?output directory}"
mkdir -p "$OUT"
ROCM="${ROCM_PATH:-/opt/rocm}"
CSRC="$ROOT/flow_matching_diffusion_amd/csrc"
OBJ="$ROOT/flow_matching_diffusion_amd/_build"
FLAGS=(-O1 -g -std=c++17 -fPIC --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops
       -I"$ROOT/include" -I"$CSRC")
SAN=(-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer
     -Xarch_host -fno-sanitize-recover=undefined)
"$ROCM/bin/hipcc" -x hip "${FLAGS[@]}" "${SAN[@]}" -c "$CSRC/k2_api.cpp" -o "$OUT/k2_api_san.o"
"$ROCM/bin/hipcc" "${FLAGS[@]}" "${SAN[@]}" -I"$ROOT/include" -c "$HERE/abi_host_checks.cpp" -o "$OUT/checks.o"
"$ROCM/bin/hipcc" --offload-arch=gfx950 "${SAN[@]}" "$OUT/checks.o" "$OUT/k2_api_san.o" \
  "$OBJ/gemm.o" "$OBJ/attention.o" "$OBJ/elementwise.o" "$OBJ/backward.o" "$OBJ/probe.o" -o "$OUT/abi_host_checks"
ASAN_OPTIONS=detect_leaks=0:abort_on_error=1 UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1 "$OUT/abi_host_checks"
