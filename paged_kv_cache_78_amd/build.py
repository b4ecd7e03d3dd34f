"""Build libpa.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m paged_kv_cache_78_amd.build        # or build() from Python

Each csrc/*.hip file is compiled to an object with hipcc (csrc/*.cpp, host
code only, with g++), in parallel, and the objects are linked into
paged_kv_cache_78_amd/libpa.so.  hipcc cross-compiles,
so this works on a machine without a GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")
PROBE = os.path.join(PKG, "probe")
PROBE_LIB = os.path.join(PKG, "libpa_probe.so")
ARCH = "gfx950"


def _hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function",
    # packed fp32 vector ops (v_pk_*_f32) are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# host-only C++ (the block manager): the system C++ compiler
HOST = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str, tag: str = "") -> str:
    obj = os.path.join(OBJ, tag + os.path.splitext(os.path.basename(src))[0] + ".o")
    if src.endswith(".cpp"):
        cmd = [shutil.which("g++") or "g++", *HOST, "-c", src, "-o", obj]
    else:
        cmd = [_hipcc(), *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    # every symbol resolved at link time: a kernel whose launch stub the host
    # pass failed to emit must fail the build, not the first load
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp,
           *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """libpa.so (the library) and libpa_probe.so (the streaming probe bench.py
    reads the HBM ceiling with)."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    probe_srcs = sorted(os.path.join(PROBE, f) for f in os.listdir(PROBE) if f.endswith(".hip"))
    jobs = [(s, "") for s in srcs] + [(s, "probe_") for s in probe_srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
