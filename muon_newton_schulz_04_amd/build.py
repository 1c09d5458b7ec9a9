"""Compiles the HIP library for gfx950 into muon_newton_schulz_04_amd/lib/.

    python -m muon_newton_schulz_04_amd.build        (or __graft_entry__.build())

Every call recompiles. The kernels are built with packed-fp32 instruction
selection switched off.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
OBJDIR = os.path.join(PKG, "_build")
LIBNAME = "libmuon_mi355x.so"
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the Muon library)")


def rocm_include() -> str:
    root = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(root, "include")


COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{os.path.join(os.path.dirname(PKG), 'include')}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
SOURCES = [("kernels.hip", True), ("adam.hip", True), ("noalloc.hip", True), ("api.cpp", False),
           ("plan.cpp", False)]


def run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(LIBDIR, exist_ok=True)
    os.makedirs(OBJDIR, exist_ok=True)
    objs = []
    for src, device in SOURCES:
        obj = os.path.join(OBJDIR, src + ".o")
        cmd = [cc, *COMMON]
        if device:
            cmd += DEVICE + ["-x", "hip"]
        else:
            cmd += ["-x", "c++", "-D__HIP_PLATFORM_AMD__", f"-I{rocm_include()}"]
        cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd))
        run(cmd)
        objs.append(obj)
    tmp = os.path.join(LIBDIR, LIBNAME + ".tmp")
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd))
    run(cmd)
    final = os.path.join(LIBDIR, LIBNAME)
    os.replace(tmp, final)
    return final


if __name__ == "__main__":
    print(build(verbose=True))
