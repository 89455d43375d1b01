"""Build libbsa.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python block_sparse_attention_antidiagonal_amd/build.py

Every HIP source is compiled with hipcc for gfx950 only; the host helpers are plain C++.
Packed fp32 instruction selection is disabled for all device code.  Device code is compiled
assuming no NaN operands (inputs are finite; the kernels produce -inf but never NaN), which
lets max/min skip NaN quieting.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbsa.so")
ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Device code assumes no NaN inputs (max/min skip NaN quieting); host validation keeps
    # full IEEE semantics.  (The hardware IEEE mode stays on: turning it off keeps the device
    # library's work-item and work-group queries from being inlined.)
    "-Xarch_device", "-fno-honor-nans",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}", f"-I{ROCM}/include"]


def _sources():
    files = sorted(os.listdir(CSRC))
    hip = [os.path.join(CSRC, f) for f in files if f.endswith(".hip")]
    cpp = [os.path.join(CSRC, f) for f in files if f.endswith(".cpp")]
    return hip, cpp


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature; that warning is noise.
    err = "\n".join(line for line in res.stderr.splitlines() if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libbsa.so next to this file; returns its path."""
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    cxx = shutil.which("g++") or "g++"
    os.makedirs(OUT_DIR, exist_ok=True)
    hip, cpp = _sources()
    cmds, objs = [], []
    for src in hip:
        obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
        cmds.append([hipcc, *HIP_FLAGS, "-c", src, "-o", obj])
        objs.append(obj)
    for src in cpp:
        obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
        cmds.append([cxx, *CXX_FLAGS, "-c", src, "-o", obj])
        objs.append(obj)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
