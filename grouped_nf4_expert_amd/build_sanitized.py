"""Build libgnf4.so with AddressSanitizer and UndefinedBehaviorSanitizer on
its HOST code (argument checks, planners, launch code); device code is
compiled as in the normal build.  For CPU runs of the host-side tests:

    python -m grouped_nf4_expert_amd.build_sanitized
    LD_PRELOAD=$(/opt/rocm/lib/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so) \\
        ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \\
        python -m pytest tests/test_library.py tests/test_ceilings.py -q -m "not gpu"

The interpreter is not instrumented, so the sanitizer runtime is preloaded;
leak detection is off because the interpreter itself never frees some of
its allocations.  Rebuild with `python -m grouped_nf4_expert_amd.build`
afterwards.
"""

import sys

from grouped_nf4_expert_amd import build as _b

HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
LINK_SANITIZE = ["-shared-libasan", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                 "-fsanitize=undefined"]


if __name__ == "__main__":
    _b.build(verbose=True, extra_compile=HOST_SANITIZE, extra_link=LINK_SANITIZE, timeline=False)
    sys.exit(0)
