"""Build libgq.so (the C-ABI library) in-tree with hipcc for gfx950.

Every .hip file under csrc/ is compiled to an object in parallel, then
linked into ``gguf_block_quant_gq_amd/libgq.so``. Compiled with -O3, no
fast-math, no denormal flushing, and with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build", "gq")
LIB = os.path.join(HERE, "libgq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
    f"-I{os.path.join(ROOT, 'include')}",
]


# The sanitizer build (host code only: the GPU code is unchanged) goes to
# _build/gq-san/libgq.so; tests/sanitize.py loads it in a process that has the
# clang address-sanitizer runtime preloaded.
SAN_OBJ = os.path.join(ROOT, "_build", "gq-san")
SAN_LIB = os.path.join(SAN_OBJ, "libgq.so")
SAN_FLAGS = [
    "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
]


def _stale(src: str, obj: str) -> bool:
    """True when obj is missing or older than src or any header under csrc/."""
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    deps = [src, *glob.glob(os.path.join(CSRC, "*.h")), os.path.join(ROOT, "include", "gq.h")]
    return any(os.path.getmtime(d) > t for d in deps if os.path.exists(d))


def _compile(src: str, verbose: bool, incremental: bool = False, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_OBJ if sanitize else OBJ, os.path.basename(src) + ".o")
    if incremental and not _stale(src, obj):
        return obj
    cmd = [HIPCC, *CFLAGS, *(SAN_FLAGS if sanitize else []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg, flush=True)
    return obj


def build(verbose: bool = False, incremental: bool = False, sanitize: bool = False) -> str:
    """Compile every HIP source and link libgq.so. With incremental=True,
    objects newer than their source and every header are reused. With
    sanitize=True the host code is built with address and undefined-behaviour
    sanitizers into SAN_LIB (the in-tree library is left alone)."""
    out_dir, lib = (SAN_OBJ, SAN_LIB) if sanitize else (OBJ, LIB)
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, incremental, sanitize), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


# The plain C client of the C ABI (tests/c_client.c): gcc, C11, linked
# against libgq.so (found next to the package through the run path) and the
# HIP runtime. The binary sits beside its source and is git-ignored.
C_CLIENT_SRC = os.path.join(ROOT, "tests", "c_client.c")
C_CLIENT = os.path.join(ROOT, "tests", "gq_c_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_client(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror",
           "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROCM, 'include')}",
           f"-I{os.path.join(ROOT, 'include')}", C_CLIENT_SRC, "-o", C_CLIENT + ".tmp",
           f"-L{HERE}", "-lgq", f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../gguf_block_quant_gq_amd", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed for {C_CLIENT_SRC}:\n{r.stdout}{r.stderr}")
    os.replace(C_CLIENT + ".tmp", C_CLIENT)
    return C_CLIENT


if __name__ == "__main__":
    import sys
    print(build(verbose=True, incremental="--incremental" in sys.argv, sanitize="--sanitize" in sys.argv))
