"""Build libmla_decode.so (gfx950 HIP kernels + C ABI) in the package directory.

Run as a script (``python mla_latent_decode_absorbed_amd/build.py``) or load it
by file path: importing it as a submodule would first run the package's
``__init__``, which refuses to import while the library is not built yet.
"""
from __future__ import annotations

import importlib.util
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmla_decode.so")
SOURCES = [os.path.join(CSRC, "mla_kernels.hip"), os.path.join(CSRC, "mla_qprep.hip"),
           os.path.join(CSRC, "mla_upproj.hip"), os.path.join(CSRC, "mla_gather.hip"),
           os.path.join(CSRC, "mla_scratch.hip"), os.path.join(CSRC, "mla_api.cpp")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU ops stay off (plain float code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def check_wait_states(verbose: bool = False) -> None:
    """Compile the kernels to gfx950 assembly and verify the wait states around
    the inline-assembly MFMAs (see isa_check.py); raises on a violation."""
    spec = importlib.util.spec_from_file_location("_mla_isa_check", os.path.join(PKG, "isa_check.py"))
    isa_check = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(isa_check)
    asm = os.path.join(PKG, "_kernels_gfx950.s")
    flags = [f for f in HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [hipcc(), *flags, "--cuda-device-only", "-S", "-I", INCLUDE, "-I", CSRC, "-o", asm, SOURCES[0]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc -S failed with status {res.returncode}")
    try:
        problems = isa_check.check_asm(open(asm).read())
    finally:
        os.remove(asm)
    if problems:
        raise RuntimeError("gfx950 wait-state check failed:\n  " + "\n  ".join(problems[:20]))
    if verbose:
        print("wait-state check: ok", flush=True)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 into the package's libmla_decode.so (always
    rebuilds), after checking the wait states of the generated kernel code."""
    check_wait_states(verbose)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
