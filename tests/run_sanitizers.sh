#!/bin/bash
# Host-side sanitizer passes over the CPU test suite (no GPU needed).
#   1. the oracle built with gcc -fsanitize=address,undefined, loaded by every
#      oracle-using CPU test (SPEC_ORACLE_LIB), with gcc's runtimes preloaded;
#   2. libspec's host code (the C ABI: argument checks, planning, K choice)
#      built with clang's -fsanitize=address,undefined on the host pass only,
#      loaded by the ABI and K-choice tests (SPEC_LIBSPEC), with clang's
#      runtime preloaded.
# Each pass preloads one sanitizer runtime, so the two run as separate
# processes.  Any sanitizer report makes the pass exit non-zero.
set -euo pipefail
cd "$(dirname "$0")/.."
python -m oracle.build --sanitize > /dev/null
python -m speculative_decoding_02_amd.build > /dev/null          # kernel objects the sanitized link reuses
python -m speculative_decoding_02_amd.build --sanitize > /dev/null
export ASAN_OPTIONS=detect_leaks=0:abort_on_error=1:halt_on_error=1
export UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1
loaded() {  # which build of $1 a process with this environment loads
  python - "$1" <<'PY'
import sys
if sys.argv[1] == "oracle":
    import oracle; oracle.lib()
else:
    import speculative_decoding_02_amd as sd; sd.binding.lib()
print(sorted({l.split()[-1] for l in open("/proc/self/maps") if "liboracle" in l or "libspec" in l}))
PY
}
echo "pass 1: oracle (gcc ASan + UBSan) under the CPU tests"
LD_PRELOAD="$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so)" \
  SPEC_ORACLE_LIB=_build/sanitize/liboracle.so loaded oracle
LD_PRELOAD="$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so)" \
  SPEC_ORACLE_LIB=_build/sanitize/liboracle.so \
  python -m pytest tests -q -m "not gpu" -p no:cacheprovider
echo "pass 2: libspec host code (clang ASan + UBSan) under the ABI and K-choice tests"
LD_PRELOAD="$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so)" \
  SPEC_LIBSPEC=_build/sanitize/libspec.so loaded libspec
LD_PRELOAD="$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so)" \
  SPEC_LIBSPEC=_build/sanitize/libspec.so \
  python -m pytest tests/test_abi.py tests/test_choose_k.py -q -p no:cacheprovider
echo "sanitizer passes clean"
