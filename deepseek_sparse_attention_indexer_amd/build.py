"""Build libdsa.so in-tree with hipcc for gfx950 (python deepseek_sparse_attention_indexer_amd/build.py).

Every source compiles to its own object in parallel (a few hipcc processes at once), then one
link step makes the shared library.

build(asan=True) makes a copy whose host code (argument checks, workspace carving, launch
policies) is built with AddressSanitizer, for the CPU tests of the C ABI: the GPU code is
compiled as usual, and the sanitizer's runtime is not linked in (the process that loads the
library preloads it; asan_runtime() names it).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # never let the compiler emit packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # fp32 denormals are preserved (the default, stated): exact fnuz e4m3 decoding relies on it
    "-fno-gpu-flush-denormals-to-zero",
]


def sources(src_dir: str | None = None) -> list[str]:
    return sorted(glob.glob(os.path.join(src_dir or os.path.join(HERE, "csrc"), "*.hip")))


# host code only: each sanitizer flag is bound to the host compilation
ASAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The AddressSanitizer runtime of the compiler that builds the library (to preload)."""
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise FileNotFoundError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm/lib/clang")
    return found[-1]


def build(verbose: bool = False, src_dir: str | None = None, out: str | None = None,
          extra_flags: tuple[str, ...] = (), asan: bool = False) -> str:
    out = out or os.path.join(HERE, "libdsa.so")
    if asan:
        extra_flags = tuple(extra_flags) + tuple(ASAN_HOST_FLAGS)
    obj_dir = os.path.join(os.path.dirname(out), "_build_asan" if asan else "_build")
    os.makedirs(obj_dir, exist_ok=True)
    inc = "-I" + os.path.join(ROOT, "include")

    def compile_one(src: str) -> str:
        obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
        cmd = ["hipcc", *HIPCC_FLAGS, *extra_flags, inc, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed compiling {os.path.basename(src)}")
        return obj

    srcs = sources(src_dir)
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "8")), 16))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = out + ".tmp"
    # -z defs: a symbol left undefined (e.g. a kernel whose host stub was not emitted) fails
    # the link here instead of the first load of the library (not for the sanitized copy, whose
    # sanitizer symbols come from the preloaded runtime)
    defs = [] if asan else ["-Wl,-z,defs"]
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *defs, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed linking libdsa.so")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
