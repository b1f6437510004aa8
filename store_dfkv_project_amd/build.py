"""Build libdfkv.so in-tree with hipcc for gfx950 (MI355X)."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdfkv.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libdfkv needs the ROCm toolchain")


def command(out: str = LIB, defines=(), sanitize: bool = False) -> list:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    # sanitize: the host code (validation, planning, dispatch) with AddressSanitizer and
    # UndefinedBehaviorSanitizer; the GPU code is built as always
    san = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"] if sanitize else []
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", *san,
            *[f"-D{d}" for d in defines],
            # packed fp32 instructions are kept out of every kernel (hipcc's host pass
            # warns that it does not know the feature; that is expected)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-result", *srcs, "-o", out]


def build(out: str = LIB, verbose: bool = False, defines=(), sanitize: bool = False) -> str:
    tmp = out + ".tmp"
    cmd = command(tmp, defines, sanitize)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libdfkv")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
