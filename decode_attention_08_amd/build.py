"""Build the HIP libraries in-tree beside this file: ``libgqa_decode.so`` (the
decode path) and ``libhbm_probe.so`` (a streaming-read probe that only the
benchmark loads).

Compiles for gfx950 only.  Packed-fp32 VALU instructions are disabled for the
device code (the host pass warns that it does not know the feature; that is
harmless).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "gqa_decode.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgqa_decode.so")
PROBE_SRC = os.path.join(HERE, "csrc", "hbm_read_probe.hip")
PROBE_LIB = os.path.join(HERE, "libhbm_probe.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the library)")


def command(out: str = LIB, src: str = SRC) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Werror=return-type",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", src, "-o", out]


def _compile(src: str, lib: str, verbose: bool) -> str:
    tmp = lib + ".tmp"
    cmd = command(tmp, src)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile both libraries (always, even when built copies exist); return the
    decode library's path."""
    _compile(PROBE_SRC, PROBE_LIB, verbose)
    return _compile(SRC, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
