"""Build the gfx950 HIP library kv_reuse_amd/libmac.so (kernels + C-ABI runtime).

Run as ``python -m kv_reuse_amd.build``.  Compiles for gfx950 only, with the
packed-fp32 instruction forms disabled.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmac.so")
SOURCES = ["match.hip", "complete.hip", "reduce.hip", "amend.hip", "prefill.hip", "mac_runtime.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False, save_temps: str = "") -> str:
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-result",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    if save_temps:
        cmd += ["-save-temps=obj", "-Rpass-analysis=kernel-resource-usage"]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    cmd += ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=save_temps or None)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
