#!/bin/bash
# Builds tests/native/_build/abi_exercise: the library sources and the ABI
# exercise driver with AddressSanitizer and UndefinedBehaviorSanitizer on the
# host code only (each -fsanitize= sits behind -Xarch_host; the gfx950 device
# code is compiled as in the library build, without sanitizers).  The objects
# are linked statically into one executable, so the sanitizer runtime is part
# of the program.  Run it on a machine with an MI355X:
#   ASAN_OPTIONS=detect_leaks=0:halt_on_error=1:verify_asan_link_order=0 \
#   UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 tests/native/_build/abi_exercise
# detect_leaks=0: the HIP runtime keeps allocations until exit by design.
set -euo pipefail
HERE="$(cd "$(dirname "${BASH_SOURCE[0]}")" && pwd)"
ROOT="$(cd "$HERE/../.." && pwd)"
CSRC="$ROOT/soft_clustering_amd/csrc"
OUT="$HERE/_build"
mkdir -p "$OUT"
HIPCC=/opt/rocm/bin/hipcc
CLANG=/opt/rocm/llvm/bin/clang++
# -O3 and the target features of the library build, so the device code is the same
COMMON=(--offload-arch=gfx950 -O3 -std=c++17 -I "$ROOT/include"
        -Xclang -target-feature -Xclang -packed-fp32-ops)
SAN=(-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined
     -Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer -Xarch_host -g)
# an object is rebuilt when it is missing or older than its source or a header
stale() {
  local o="$1" s="$2" h
  [ -s "$o" ] || return 0
  for h in "$s" "$CSRC"/*.h "$ROOT"/include/*.h; do [ "$h" -nt "$o" ] && return 0; done
  return 1
}
objs=()
for src in gmm_kernels gmm_assign gmm_lists gmm_api; do
  if stale "$OUT/$src.o" "$CSRC/$src.hip"; then
    rm -f "$OUT/$src.o"
    "$HIPCC" "${COMMON[@]}" "${SAN[@]}" -c "$CSRC/$src.hip" -o "$OUT/$src.o" 2> "$OUT/$src.log" &
  fi
  objs+=("$OUT/$src.o")
done
if stale "$OUT/abi_exercise.o" "$HERE/abi_exercise.cpp"; then
  rm -f "$OUT/abi_exercise.o"
  "$HIPCC" "${COMMON[@]}" "${SAN[@]}" -x hip -c "$HERE/abi_exercise.cpp" -o "$OUT/abi_exercise.o" \
    2> "$OUT/abi_exercise.log" &
fi
wait
for o in "${objs[@]}" "$OUT/abi_exercise.o"; do
  [ -s "$o" ] || { echo "compile failed: $o" >&2; grep -i error "${o%.o}.log" >&2; exit 1; }
done
# host link: objects only, the sanitizer runtimes linked statically
"$CLANG" -fsanitize=address,undefined -o "$OUT/abi_exercise" "$OUT/abi_exercise.o" "${objs[@]}" \
  -L/opt/rocm/lib -Wl,-rpath,/opt/rocm/lib -lamdhip64
echo "built $OUT/abi_exercise"
