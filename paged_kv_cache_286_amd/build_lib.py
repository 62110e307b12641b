"""Build libpagedkv.so (HIP for gfx950 only) in place, next to this file.

    python -m paged_kv_cache_286_amd.build_lib

Every ``csrc/*.hip`` (device and host) and ``csrc/*.cpp`` (host only) file is
compiled by hipcc into ``_build/`` in parallel and the objects are linked into
``libpagedkv.so``; ``libpagedkv_checks.so`` links the same objects with
``api.hip`` compiled again with ``PKV_CHECKS`` (contract checks of the attention
step's metadata, for debugging).  The build always runs
(no staleness check), so a changed source is always picked up.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpagedkv.so")
# the same library with the contract checks of paged_attn_step compiled in
CHECKS_LIB = os.path.join(HERE, "libpagedkv_checks.so")
# the one source the checks build compiles differently
CHECKS_SRC = "api.hip"
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


# Per-file additions.  The MFMA tile kernels never compute with a NaN (slots
# past a context or outside the pool read as zeros, masked scores are selected
# to -inf), so they are compiled without NaN semantics: every fmaxf after a
# cross-lane swap otherwise carries an extra v_max that only quiets NaNs
# (8 of the 146 vector instructions of a prefill tile's block pair).
FILE_FLAGS = {"tile_mfma.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def _compile(src: str, checks: bool = False) -> str:
    stem = os.path.splitext(os.path.basename(src))[0] + ("_checks" if checks else "")
    obj = os.path.join(BUILD, stem + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []),
           *(["-DPKV_CHECKS"] if checks else []),
           "-I", os.path.join(HERE, "..", "include"), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    checks_src = os.path.join(CSRC, CHECKS_SRC)
    jobs = max(1, min(8, len(srcs) + 1, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(jobs) as ex:
        fut_checks = ex.submit(_compile, checks_src, True)
        objs = list(ex.map(_compile, srcs))
        obj_checks = fut_checks.result()
    for lib, lib_objs in ((LIB, objs),
                          (CHECKS_LIB, [obj_checks if s == checks_src else o
                                        for s, o in zip(srcs, objs)])):
        tmp = lib + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *lib_objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(tmp, lib)
        if verbose:
            print(f"built {lib} from {len(srcs)} sources", flush=True)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
