"""Build the StagQ HIP library (libstagq.so) in-tree for gfx950.

    python -m precision_weight_only_amd.build [--verbose]

Compiles every source under csrc/ with hipcc into one shared library next to
this file.  Packed-FP32 instructions are disabled for the device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libstagq.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = [ln for ln in (res.stdout + res.stderr).splitlines()
           if "packed-fp32-ops' is not a recognized feature" not in ln]
    if res.returncode != 0:
        raise RuntimeError("build step failed: " + " ".join(cmd) + "\n" + "\n".join(out))
    if verbose and out:
        print("\n".join(out))


def build_library(verbose: bool = False, extra_flags=()) -> str:
    """Compile the host packer/encoder with g++ and the kernels with hipcc, link with hipcc."""
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    tmpdir = tempfile.mkdtemp(prefix="stagq_build_")
    try:
        host_o = os.path.join(tmpdir, "stagq_host.o")
        dev_o = os.path.join(tmpdir, "stagq_device.o")
        _run(["g++", "-O3", "-std=c++17", "-fPIC", "-Wall", "-pthread", *inc,
              "-c", os.path.join(CSRC, "stagq_host.cpp"), "-o", host_o], verbose)
        _run([hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
              *inc, *extra_flags, "-c", os.path.join(CSRC, "stagq_device.hip"), "-o", dev_o], verbose)
        fd, tmp = tempfile.mkstemp(suffix=".so", dir=HERE)
        os.close(fd)
        try:
            _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread",
                  host_o, dev_o, "-o", tmp], verbose)
            os.replace(tmp, LIB)
        finally:
            if os.path.exists(tmp):
                os.unlink(tmp)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="--verbose" in sys.argv))
