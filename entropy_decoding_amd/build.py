"""Builds libdf11.so in-tree: host codec with g++, gfx950 kernels with hipcc."""

from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdf11.so")

ARCH = "gfx950"
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# packed fp32 instructions are kept off in all device code
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-command-line-argument"]
CXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-pthread", "-Wall", "-Wextra"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def build_library(verbose: bool = False, extra_hip_flags=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    host_o = os.path.join(BUILD, "df11_host.o")
    dev_o = os.path.join(BUILD, "df11_device.o")
    _run(["g++", *CXX_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, "df11_host.cpp"),
          "-o", host_o], verbose)
    _run([HIPCC, *HIP_FLAGS, *extra_hip_flags, "-I", INCLUDE, "-c",
          os.path.join(CSRC, "df11_device.hip"), "-o", dev_o], verbose)
    objs = [host_o, dev_o]
    for name in ("df11_pipeline", "df11_encode_device"):
        o = os.path.join(BUILD, name + ".o")
        _run([HIPCC, *HIP_FLAGS, *extra_hip_flags, "-I", INCLUDE, "-c",
              os.path.join(CSRC, name + ".hip"), "-o", o], verbose)
        objs.append(o)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-pthread", "-o", tmp],
         verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
