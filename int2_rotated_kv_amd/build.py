"""Build liboscar.so (HIP, gfx950) in-tree with hipcc.

    python -m int2_rotated_kv_amd.build [--jobs N] [--debug]

Every translation unit under csrc/ is compiled for gfx950 and linked into
int2_rotated_kv_amd/liboscar.so next to this file.  With --debug the same
sources are built with OSCAR_DEBUG (kernels report indices they would clamp
or skip through the cache's status word, OSCAR_STATUS_DEBUG_BOUNDS) into
liboscar_debug.so; the binding loads it when OSCAR_LIB names it.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "liboscar.so")
LIB_DEBUG = os.path.join(HERE, "liboscar_debug.so")

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def common_flags(debug: bool = False):
    f = [f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-I", INCLUDE, "-I", CSRC,
         # packed fp32 VALU instructions are disabled on purpose for all device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-munsafe-fp-atomics",
         # keep matrix-core accumulators in VGPRs: the online-softmax rescale
         # multiplies them with VALU ops, which cannot read AGPRs
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         # keep uniform-address atomics as written: the optimiser's lane
         # aggregation waits for each result right after issuing it
         "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]
    f += ["-O2", "-g", "-DOSCAR_DEBUG"] if debug else ["-O3"]
    return f


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def compile_one(src: str, debug: bool) -> str:
    bdir = os.path.join(BUILD, "debug") if debug else BUILD
    os.makedirs(bdir, exist_ok=True)
    obj = os.path.join(bdir, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags(debug) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l and l.strip() and "warning generated" not in l)
    if warn:
        print(warn, file=sys.stderr)
    return obj


def build(jobs: int = 8, debug: bool = False, verbose: bool = True) -> str:
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: compile_one(s, debug), srcs))
    lib = LIB_DEBUG if debug else LIB
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources")
    return lib


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--debug", action="store_true")
    a = ap.parse_args(argv)
    build(a.jobs, a.debug)


if __name__ == "__main__":
    main()
