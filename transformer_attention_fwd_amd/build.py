"""Build libfa.so (HIP kernels + C-ABI entry point) for gfx950, in place next to this file."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
SOURCES = [os.path.join(CSRC, f) for f in ("fa_kernels.hip", "fa_merge.hip", "fa_bwd.hip", "fa_bwd32.hip", "fa_api.cpp")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    # no packed fp32 VALU ops (v_pk_{add,mul,fma}_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    """Compile every source into libfa.so (always recompiles).  Returns the library path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS
    for src in SOURCES:
        cmd += ["-x", "hip", src]
    cmd += ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
