"""Build libpkd.so (HIP kernels for gfx950 + host scheduler + C ABI) in-tree.

    python -m paged_kv_decode_11_amd.build [--verbose]

Kernels are compiled with hipcc for gfx950 only, with packed-fp32 VALU
instructions disabled.  The host scheduler is plain C++17 and the C ABI
host code uses only the HIP runtime API.  Output: paged_kv_decode_11_amd/libpkd.so.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpkd.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
KERNEL_SOURCES = ["decode.hip", "decode_mfma.hip", "decode_pv.hip", "decode_fp8.hip", "merge.hip",
                  "upload.hip", "prefix_mfma.hip", "append.hip", "read_ceiling.hip",
                  "static_scratch.hip", "composable.hip"]
HOST_SOURCES = ["plan.cpp", "api.cpp"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def compile_commands():
    cmds = []
    objs = []
    for src in KERNEL_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        cmds.append([HIPCC, "-c", *COMMON, *DEVICE, os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        cmds.append([HIPCC, "-x", "c++", "-c", *COMMON, "-D__HIP_PLATFORM_AMD__",
                     "-I", os.path.join(ROCM, "include"), os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    link = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", LIB + ".tmp",
            f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    return cmds, link


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    cmds, link = compile_commands()
    with ThreadPoolExecutor(max_workers=min(4, len(cmds))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    _run(link, verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
