"""Build libdsa.so in-tree with hipcc for gfx950 (python deepseek_sparse_attention_indexer_amd/build.py).

Every source compiles to its own object in parallel (a few hipcc processes at once), then one
link step makes the shared library.
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


def build(verbose: bool = False, src_dir: str | None = None, out: str | None = None,
          extra_flags: tuple[str, ...] = ()) -> str:
    out = out or os.path.join(HERE, "libdsa.so")
    obj_dir = os.path.join(os.path.dirname(out), "_build")
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
    # the link here instead of the first load of the library
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
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
