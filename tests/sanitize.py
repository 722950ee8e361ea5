"""Run the CPU test suite (-m "not gpu") against sanitizer builds.

Builds the oracle with clang's address and undefined-behaviour sanitizers
(oracle/libgq_oracle_san.so, selected by GQ_SANITIZE=1) and the host code of
the C-ABI library with the same sanitizers (_build/gq-san/libgq.so, selected
by GQ_LIBRARY), then runs pytest in a child process with the sanitizer
runtime preloaded (the Python interpreter itself is not instrumented).
Leak detection is off: the interpreter and the HIP runtime keep allocations
until exit by design. Any sanitizer report aborts the run with a non-zero
status.

    python tests/sanitize.py [extra pytest arguments]
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def runtime() -> str:
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not libs:
        raise SystemExit("clang address-sanitizer runtime not found under /opt/rocm/llvm")
    return libs[-1]


def main() -> int:
    sys.path.insert(0, ROOT)
    env = dict(os.environ)
    env["GQ_SANITIZE"] = "1"
    # build both instrumented libraries in this (uninstrumented) process
    build = ("import oracle, gguf_block_quant_gq_amd._build as b; "
             "oracle.build(verbose=True); print(b.build(incremental=True, sanitize=True))")
    subprocess.run([sys.executable, "-c", build], cwd=ROOT, env=env, check=True)
    from gguf_block_quant_gq_amd import _build
    env["GQ_LIBRARY"] = _build.SAN_LIB
    env["LD_PRELOAD"] = runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests"), *sys.argv[1:]]
    print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


if __name__ == "__main__":
    sys.exit(main())
