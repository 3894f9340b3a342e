"""CPU sanitizer run: builds AddressSanitizer + UndefinedBehaviorSanitizer versions of the oracle
(oracle/moe_oracle.c), the host input generator (synth/synth_host.c) and the C-ABI library's host
code (its argument and dtype-tag validation, handle and JIT bookkeeping; device code is compiled as
usual, not instrumented), then runs the CPU test suite (-m "not gpu") with them loaded in place of
the normal builds.  Any sanitizer report ends the run with an error.

    python tests/sanitized.py [extra pytest arguments]

The builds go to _build/san/ at the repository root; the loaders take them from there when
MOE_SANITIZED_LIBS names that directory.  All three are built with ROCm's clang and its shared
sanitizer runtime, which is preloaded into the Python process (Python itself is not instrumented).
Leak checking is off: the interpreter and the HIP runtime hold memory until exit by design.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "san")
LLVM = "/opt/rocm/llvm"
CLANG = os.path.join(LLVM, "bin", "clang")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g",
       "-shared-libsan"]


def runtime() -> str:
    libs = glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    if not libs:
        raise RuntimeError("ROCm clang's shared AddressSanitizer runtime was not found")
    return libs[0]


def _fresh(outputs, inputs) -> bool:
    """Every output exists and is newer than every input."""
    if not all(os.path.exists(o) for o in outputs):
        return False
    return min(os.path.getmtime(o) for o in outputs) > max(os.path.getmtime(i) for i in inputs)


def build() -> None:
    os.makedirs(OUT, exist_ok=True)
    inputs = (glob.glob(os.path.join(ROOT, "oracle", "*.c")) + glob.glob(os.path.join(ROOT, "synth", "*.c")) +
              [f for f in glob.glob(os.path.join(ROOT, "mxfp4_expert_gemv_amd", "csrc", "*"))
               if not f.endswith("moe_jit_sources.h")] +  # generated from the headers listed here
              glob.glob(os.path.join(ROOT, "include", "*.h")) + [os.path.abspath(__file__)])
    outputs = [os.path.join(OUT, n) for n in ("libmoe_oracle.so", "libsynth_host.so", "libmoe_decode.so")]
    if _fresh(outputs, inputs):
        return
    c_flags = ["-O1", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-shared", "-fPIC", *SAN]
    subprocess.check_call([CLANG, *c_flags, "-fopenmp", f"-Wl,-rpath,{LLVM}/lib",
                           os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", os.path.join(OUT, "libmoe_oracle.so"),
                           "-lm"])
    subprocess.check_call([CLANG, *c_flags, os.path.join(ROOT, "synth", "synth_host.c"),
                           "-o", os.path.join(OUT, "libsynth_host.so"), "-lm"])
    sys.path.insert(0, ROOT)
    from mxfp4_expert_gemv_amd import build as pkg
    import __graft_entry__ as entry
    pkg.write_jit_sources()
    host = []
    for f in SAN:  # host code only: every sanitizer flag is scoped to the host compilation
        host += ["-Xarch_host", f]
    flags = [f for f in entry.HIP_FLAGS if f != "-O3"] + ["-O1"] + host
    subprocess.check_call([HIPCC, *flags, *pkg.SOURCES, "-o", os.path.join(OUT, "libmoe_decode.so"), "-lhiprtc"],
                          cwd=os.path.dirname(pkg.__file__))


def main() -> int:
    build()
    env = dict(os.environ)
    env["MOE_SANITIZED_LIBS"] = OUT
    env["LD_PRELOAD"] = runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    # the given test files or options, else the whole CPU suite (this script's own test excluded)
    targets = sys.argv[1:] or [os.path.join(ROOT, "tests"), "--deselect",
                               "tests/test_sanitizers.py::test_abi_and_oracle_pins_under_asan_and_ubsan"]
    cmd = [sys.executable, "-m", "pytest", "-m", "not gpu", "-q", "-x", "-p", "no:cacheprovider", *targets]
    return subprocess.call(cmd, cwd=ROOT, env=env)


if __name__ == "__main__":
    sys.exit(main())
