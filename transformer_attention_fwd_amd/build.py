"""Build libfa.so (HIP kernels + C-ABI entry point) for gfx950, in place next to this file.

Also builds libfa_tilecount.so, a test-only variant of the same sources compiled with FA_TILE_COUNT: its
forward kernels record the K/V tiles every workgroup visits (tests/test_gpu_tile_visits.py).  The product
path loads libfa.so only.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
LIB_TILECOUNT = os.path.join(HERE, "libfa_tilecount.so")
SOURCES = [os.path.join(CSRC, f) for f in ("fa_kernels.hip", "fa_merge.hip", "fa_bwd.hip", "fa_bwd32.hip", "fa_api.cpp")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    # no packed fp32 VALU ops (v_pk_{add,mul,fma}_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _command(out: str, extra: list[str]) -> list[str]:
    cmd = [HIPCC] + FLAGS + extra
    for src in SOURCES:
        cmd += ["-x", "hip", src]
    return cmd + ["-o", out]


def build(verbose: bool = False) -> str:
    """Compile every source into libfa.so and the test-only libfa_tilecount.so (always recompiles; the two
    compilations run side by side).  Returns the path of libfa.so."""
    jobs = []
    for lib, extra in ((LIB, []), (LIB_TILECOUNT, ["-DFA_TILE_COUNT"])):
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = _command(tmp, extra)
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((lib, tmp, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for lib, tmp, proc in jobs:
        out, _ = proc.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if proc.returncode != 0:
            failed.append("hipcc failed for %s:\n%s" % (os.path.basename(lib), out))
        else:
            os.replace(tmp, lib)
    if failed:
        raise RuntimeError("\n".join(failed))
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
