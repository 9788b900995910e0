"""Compile the HIP library in-tree: csrc/*.hip -> libswiglu_gateup.so.

gfx950 only. Packed-fp32 instruction selection is switched off for the device
code (``-packed-fp32-ops``); the host pass prints a harmless warning about the
unknown feature.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
SRCS = [os.path.join(PKG_DIR, "csrc", "swiglu_gateup.hip"),
        os.path.join(PKG_DIR, "csrc", "swiglu_bias_scale.hip"),
        os.path.join(PKG_DIR, "csrc", "swiglu_fc1.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG_DIR, "libswiglu_gateup.so")
CLIENT_SRC = os.path.join(PKG_DIR, "examples", "c_abi_client.c")
CLIENT = os.path.join(PKG_DIR, "c_abi_client")       # a plain C program using the C ABI
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (needs ROCm)")


def compile_command(out: str = LIB, srcs=None, defines=()) -> list:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
           "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-I", INCLUDE]
    cmd += [f"-D{d}" for d in defines]
    cmd += ["-o", out, *(SRCS if srcs is None else srcs)]
    return cmd


def build(verbose: bool = False) -> str:
    """Compile the library (always; a stale build is never reused). Returns its path."""
    tmp = LIB + ".tmp"
    cmd = compile_command(out=tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    build_client(verbose)
    return LIB


def build_client(verbose: bool = False) -> str:
    """Compile the plain C client (C11, host compiler) against the library."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for the C ABI client")
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = [cc, "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE,
           "-I", os.path.join(rocm, "include"), "-o", CLIENT, CLIENT_SRC,
           "-L", PKG_DIR, "-lswiglu_gateup", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"C client build failed ({res.returncode}):\n{res.stderr}")
    return CLIENT


if __name__ == "__main__":
    print(build(verbose=True))
