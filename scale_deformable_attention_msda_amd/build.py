"""Builds libmsda.so (the gfx950 HIP kernels plus the C-ABI layer) in-tree."""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmsda.so")
SOURCES = ("msda_kernels.hip", "msda_api.cpp")


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libmsda.so")
    return path


def build(verbose=False, extra_flags=()):
    """Compile every source for gfx950 into scale_deformable_attention_msda_amd/libmsda.so."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed fp32 VALU forms are kept out of the generated code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", INCLUDE, "-I", CSRC, *extra_flags,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("libmsda.so build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    if verbose and res.stderr.strip():
        print(res.stderr)
    os.replace(tmp, LIB)
    return LIB


def build_c_abi_check(source, exe):
    """Compile a host program that calls the library through include/msda.h
    (HIP runtime, no torch) and links libmsda.so next to it by rpath."""
    rpath = os.path.relpath(HERE, os.path.dirname(os.path.abspath(exe)))
    cmd = [hipcc(), "-O2", "-std=c++17", "-I", INCLUDE, source, "-o", exe + ".tmp",
           "-L", HERE, "-lmsda", "-Wl,-rpath,$ORIGIN/" + rpath]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("C-ABI check program build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    os.replace(exe + ".tmp", exe)
    return exe


def build_ceiling_probes(source, exe):
    """Compile the hardware-ceiling probe program (plain HIP, no library)."""
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", source, "-o", exe + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("ceiling probe build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    os.replace(exe + ".tmp", exe)
    return exe


if __name__ == "__main__":
    print(build(verbose=True))
