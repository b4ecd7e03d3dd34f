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
# Build-flag variants of the decode kernels, kept for measurement: the same
# library with only the decode kernel files rebuilt under the flag.  Load one
# with PA_LIB=paged_kv_cache_78_amd/variants/libpa_<name>.so.
#   xlane_dpp: cross-lane reductions on DPP and v_permlane*_swap instead of
#              ds_bpermute;
#   table_lds: block-table window staged through LDS instead of v_readlane;
#   plain_grid: the vector-ALU kernel's launches past their die-order limit
#               (every launch: 3-D partition grid, one pass in index order),
#               so that the tests reach that path.
VARIANTS = {"xlane_dpp": ["-DPA_XLANE_DPP=1"], "table_lds": ["-DPA_TABLE_LDS=1"],
            "plain_grid": ["-DPA_DIE_MAX_ITEMS=0"]}
VARIANT_FILES = ("decode_valu.hip", "decode_mfma.hip")
VARIANT_DIR = os.path.join(PKG, "variants")
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


def _compile(src: str, tag: str = "", extra=()) -> str:
    obj = os.path.join(OBJ, tag + os.path.splitext(os.path.basename(src))[0] + ".o")
    if src.endswith(".cpp"):
        cmd = [shutil.which("g++") or "g++", *HOST, "-c", src, "-o", obj]
    else:
        cmd = [_hipcc(), *COMMON, *extra, "-c", src, "-o", obj]
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
    jobs = [(s, "", ()) for s in srcs] + [(s, "probe_", ()) for s in probe_srcs]
    var_srcs = [s for s in srcs if os.path.basename(s) in VARIANT_FILES]
    for name, flags in VARIANTS.items():
        jobs += [(s, name + "_", tuple(flags)) for s in var_srcs]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    base = objs[:len(srcs)]
    _link(base, LIB)
    _link(objs[len(srcs):len(srcs) + len(probe_srcs)], PROBE_LIB)
    os.makedirs(VARIANT_DIR, exist_ok=True)
    k = len(srcs) + len(probe_srcs)
    for name in VARIANTS:
        own = objs[k:k + len(var_srcs)]
        k += len(var_srcs)
        swap = dict(zip(var_srcs, own))
        _link([swap.get(s, o) for s, o in zip(srcs, base)],
              os.path.join(VARIANT_DIR, f"libpa_{name}.so"))
    if verbose:
        print(f"built {LIB}, {PROBE_LIB} and the variants in {VARIANT_DIR}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
