#!/bin/bash
# Build the host-sanitizer driver (driver.cpp) against every library source.
# Host code: AddressSanitizer + UndefinedBehaviorSanitizer (each -fsanitize=
# goes to the host compilation only, through -Xarch_host); device code: the
# library's own flags.  The driver is compiled and linked with clang++ (no
# HIP source on that line).  Usage: tests/host_sanitizer/build.sh [outdir]
# (default tests/host_sanitizer/_build); run it with
#   ASAN_OPTIONS=verify_asan_link_order=0:detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
#     tests/host_sanitizer/_build/driver
# (link order: the process may preload other libraries first; leaks: the HIP
# runtime keeps allocations until exit).
set -euo pipefail
HERE=$(cd "$(dirname "$0")" && pwd)
ROOT=$(cd "$HERE/../.." && pwd)
OUT=${1:-$HERE/_build}
CSRC=$ROOT/bit_weight_kv_amd/csrc
mkdir -p "$OUT"
pids=()
for src in elementwise quantize gemm attention runtime timing; do
  extra=()
  if [ "$src" = attention ]; then extra=(-mllvm -amdgpu-mfma-vgpr-form); fi
  /opt/rocm/bin/hipcc --offload-arch=gfx950 -O3 -std=c++17 -fPIC \
    -Xclang -target-feature -Xclang -packed-fp32-ops -fhip-fp32-correctly-rounded-divide-sqrt -Wno-unused-result \
    -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer -Xarch_host -g \
    "${extra[@]}" -I"$ROOT/include" -I"$CSRC" -c "$CSRC/$src.hip" -o "$OUT/$src.o" &
  pids+=($!)
done
for p in "${pids[@]}"; do wait "$p"; done
/opt/rocm/llvm/bin/clang++ -std=c++17 -O1 -g -fno-omit-frame-pointer -fsanitize=address,undefined \
  -I"$ROOT/include" -c "$HERE/driver.cpp" -o "$OUT/driver.o"
/opt/rocm/llvm/bin/clang++ -fsanitize=address,undefined -o "$OUT/driver" "$OUT/driver.o" \
  "$OUT"/elementwise.o "$OUT"/quantize.o "$OUT"/gemm.o "$OUT"/attention.o "$OUT"/runtime.o "$OUT"/timing.o \
  -L/opt/rocm/lib -lamdhip64 -Wl,-rpath,/opt/rocm/lib
echo "$OUT/driver"
