"""Build libfusedrow.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Each translation unit is compiled by hipcc in parallel, then linked into
memory_bound_row_pass_amd/libfusedrow.so. Only the fr_* entry points are
exported. Packed-fp32 instruction selection is disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfusedrow.so")
BUILD = os.path.join(PKG, "_build")
SOURCES = ["softmax.hip", "xent.hip", "norms.hip", "backward.hip", "split.hip", "split_norm.hip",
           "attention.hip", "copy.hip", "noalloc.hip", "mfma_probe.hip", "api.cpp"]
ARCH = os.environ.get("FR_OFFLOAD_ARCH", "gfx950")

CXXFLAGS = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


# Per-source flags. attention.hip: MFMA accumulators in VGPRs (the AGPR form
# made the compiler copy the 64 output accumulators between register files on
# every key block).
EXTRA = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(src: str, verbose: bool, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [_hipcc(), *CXXFLAGS, *EXTRA.get(src, []), *[f"-D{d}" for d in defines], *lang, "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("packed-fp32-ops", "warning: feature flag")
    err = "\n".join(l for l in r.stderr.splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if verbose and err.strip():
        print(err, flush=True)
    return obj


def build(verbose: bool = False, jobs: int | None = None, lib_path: str = LIB, defines=()) -> str:
    """Compile and link. `lib_path` and `defines` (NAME=VALUE build switches)
    produce alternative builds for A/B measurements."""
    build_dir = BUILD if lib_path == LIB else os.path.join(os.path.dirname(os.path.abspath(lib_path)), "_build")
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, defines), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
