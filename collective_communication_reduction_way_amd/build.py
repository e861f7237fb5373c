"""Build librr.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m collective_communication_reduction_way_amd.build [--jobs N]

Every translation unit is compiled by hipcc in parallel into ``_build/`` at
the repository root; the shared library lands next to this file, where the
binding loads it.  The compile never needs a GPU.
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librr.so")

ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SOURCES = [
    "rr_fold_ring_all.hip",
    "rr_fold_ring_shard.hip",
    "rr_fold_hier_all.hip",
    "rr_fold_asc_one.hip",
    "rr_copy.hip",
    "rr_multi.hip",
    "rr_exec.hip",
    "rr_scratch.hip",
    "rr_phase_ring.hip",
    "rr_phase_hier.hip",
    "rr_phase_hier_var.hip",
    "rr_phase_one.hip",
    "rr_phase.cpp",
    "rr_api.cpp",
    "rr_plan.cpp",
]

COMMON = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]
# Device code: gfx950 only; packed-fp32 instructions disabled (plain float
# code must not be turned into v_pk_* forms); no fast-math, no denormal flush.
DEVICE = [
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build librr.so")
    return path


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [hipcc(), *COMMON, *DEVICE, "-c", path, "-o", obj]
    else:
        # host-only C++: the HIP runtime API headers, no device compilation
        cmd = [hipcc(), *COMMON, "-x", "c++", f"-I{ROCM}/include", "-D__HIP_PLATFORM_AMD__", "-c", path, "-o", obj]
    t0 = time.time()
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj, time.time() - t0, res.stderr


def build(jobs=None, verbose=False):
    """Compile every source and link librr.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 4)))
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for obj, dt, err in ex.map(_compile, SOURCES):
            objs.append(obj)
            if verbose:
                print(f"  compiled {os.path.basename(obj)} in {dt:.1f}s", flush=True)
            if err.strip() and verbose:
                print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args(argv)
    t0 = time.time()
    lib = build(args.jobs, verbose=True)
    print(f"built {lib} in {time.time() - t0:.1f}s")


if __name__ == "__main__":
    main()
