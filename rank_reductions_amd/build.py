"""Builds librankred.so in-tree: host-only C++ with g++, HIP with hipcc for gfx950.

    python -m rank_reductions_amd.build        # or: python rank_reductions_amd/build.py

The session, validation and planning layers compile with the host C++ compiler
and have no HIP dependency; kernels and the launch layer compile with hipcc.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD = PKG / "_build"
LIB = PKG / "librankred.so"

HOST_SOURCES = ["session.cpp", "validate.cpp", "plan.cpp"]
# (source, object, defines): the fold and batch kernels are built once per
# element type and cache hint, so that their instantiations compile in parallel
RC_F32, RC_I32 = 0, 1
HIP_SOURCES = [
    ("kernels_fold.hip", "kernels_fold_f32_nt", {"RC_KDT": RC_F32, "RC_KNT": 1}),
    ("kernels_fold.hip", "kernels_fold_f32_cached", {"RC_KDT": RC_F32, "RC_KNT": 0}),
    ("kernels_fold.hip", "kernels_fold_i32_nt", {"RC_KDT": RC_I32, "RC_KNT": 1}),
    ("kernels_fold.hip", "kernels_fold_i32_cached", {"RC_KDT": RC_I32, "RC_KNT": 0}),
    ("kernels_batch.hip", "kernels_batch_nt", {"RC_KNT": 1}),
    ("kernels_batch.hip", "kernels_batch_cached", {"RC_KNT": 0}),
    ("kernels_copy.hip", "kernels_copy", {}),
    ("device.hip", "device", {}),
]

ARCH = "gfx950"

HOST_FLAGS = ["-std=c++17", "-O2", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter"]
HIP_FLAGS = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    # exact IEEE float32: no contraction, subnormals kept, correctly rounded division
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librankred.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(str(c) for c in cmd), flush=True)
    res = subprocess.run([str(c) for c in cmd], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(map(str, cmd))}\n"
                           f"{res.stdout}\n{res.stderr}")
    return res


def build(verbose=False, extra_hip_flags=()):
    """Compile every source and link librankred.so.  Always recompiles."""
    BUILD.mkdir(exist_ok=True)
    hipcc = _hipcc()
    cxx = os.environ.get("CXX", "g++")
    inc = [f"-I{INCLUDE}", f"-I{CSRC}"]
    jobs = []
    objs = []
    for src in HOST_SOURCES:
        obj = BUILD / (src + ".o")
        jobs.append([cxx, *HOST_FLAGS, *inc, "-c", CSRC / src, "-o", obj])
        objs.append(obj)
    for src, name, defines in HIP_SOURCES:
        obj = BUILD / (name + ".o")
        dflags = [f"-D{k}={v}" for k, v in defines.items()]
        jobs.append([hipcc, *HIP_FLAGS, *extra_hip_flags, *dflags, *inc, "-c", CSRC / src, "-o", obj])
        objs.append(obj)
    # the largest objects first, so the pool ends together
    jobs.sort(key=lambda c: 0 if "kernels_fold.hip" in str(c) else 1)
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 8, 16)) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB.with_suffix(".so.tmp")
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
