"""Build libcompkv.so (HIP for gfx950) in-tree with hipcc.

    python -m compensated_kv_selection_amd.build [-v] [--phase-trace]

Every call compiles from source; the library lands next to this file.  With
--phase-trace it builds libcompkv_trace.so instead: the same library with the
single launch's phase timestamps compiled in (CKV_PHASE_TRACE), for
compensated_kv_selection_amd.phase_trace.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libcompkv.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
TRACE_LIB_PATH = os.path.join(HERE, "libcompkv_trace.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["kernels.hip", "fused.hip", "abi.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libcompkv.so")
    return path


def _compile(src: str, verbose: bool, out_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc(), *lang, *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    return obj


def build(verbose: bool = False, phase_trace: bool = False) -> str:
    out_dir = os.path.join(BUILD_DIR, "trace") if phase_trace else BUILD_DIR
    lib_path = TRACE_LIB_PATH if phase_trace else LIB_PATH
    extra = ("-DCKV_PHASE_TRACE",) if phase_trace else ()
    os.makedirs(out_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, out_dir, extra), SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, phase_trace="--phase-trace" in sys.argv))
