"""Build step: compile the HIP sources into the in-tree shared library ``libdconv1d.so``.

Run ``python -m normalisation_dilated_conv1d_amd.build`` (or ``__graft_entry__.build()``).
hipcc cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libdconv1d.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = os.environ.get("DCONV1D_OFFLOAD_ARCH", "gfx950")

# Packed-FP32 VALU ops stay off: hipcc would otherwise form v_pk_* FP32 instructions
# from ordinary float code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build_library(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, *HIP_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


C_CLIENT_SRC = os.path.join(ROOT, "tests", "c_client", "dconv1d_client.c")
C_CLIENT_BIN = os.path.join(ROOT, "tests", "c_client", "dconv1d_client")


def build_c_client(verbose: bool = False) -> str:
    """Compile the plain C client of the ABI (tests/c_client) with gcc against the built
    library; it is run by the GPU tests."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [os.environ.get("CC", "gcc"), "-std=c99", "-O2", "-Wall", "-Wextra",
           "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}", f"-I{rocm}/include", C_CLIENT_SRC,
           f"-L{PKG}", "-ldconv1d", f"-L{rocm}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../normalisation_dilated_conv1d_amd",
           f"-Wl,-rpath,{rocm}/lib", "-o", C_CLIENT_BIN]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0 or res.stderr.strip():
        raise RuntimeError(f"C client build failed ({res.returncode}):\n{res.stderr}")
    return C_CLIENT_BIN


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_c_client(verbose=True))
