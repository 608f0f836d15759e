"""Build libpie.so (HIP kernels for gfx950 + the host engine + the C ABI) in-tree.

    python -m paged_kv_forward_amd.build [--jobs N] [--sanitize]

Every source is compiled with hipcc for gfx950 only; packed fp32 instructions
are turned off (-packed-fp32-ops) for all device code.

--sanitize builds libpie_asan.so instead: the same sources with the HOST code
instrumented by AddressSanitizer and UndefinedBehaviorSanitizer (device code
is built as usual).  It serves the host-only context path (page pool, working
sets, fork, prefix registry, batch packing) in CPU tests: load it with the
clang ASan runtime preloaded (ASAN_RUNTIME below) and PIE_LIBRARY pointing at
it.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpie.so")
LIB_ASAN = os.path.join(HERE, "libpie_asan.so")
BUILD_ASAN = os.path.join(HERE, "_build_asan")

SOURCES = ["kvstore.cpp", "packer.cpp", "engine.hip", "gemm.hip", "attention.hip", "misc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
         "-Xclang", "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
         "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


# host-side sanitizers only: each -fsanitize= goes to the host pass
SAN_FLAGS = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def asan_runtime() -> str:
    """Path of the clang ASan runtime that libpie_asan.so needs preloaded."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang ASan runtime not found under /opt/rocm/llvm")
    return hits[-1]


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD_ASAN if sanitize else BUILD, src.replace(".", "_") + ".o")
    cmd = [HIPCC] + FLAGS + (SAN_FLAGS if sanitize else []) + [
        "-x", "hip" if src.endswith(".hip") else "c++", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if errs.strip():
        sys.stderr.write(errs + "\n")
    return obj


def build(jobs: int = 0, sanitize: bool = False) -> str:
    """Compile every source and link libpie.so, or libpie_asan.so with
    sanitize (always rebuilds)."""
    os.makedirs(BUILD_ASAN if sanitize else BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    out = LIB_ASAN if sanitize else LIB
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    if sanitize:
        cmd += ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--sanitize", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.sanitize))
