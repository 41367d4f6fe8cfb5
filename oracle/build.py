"""Build the fp64 CPU oracle (test infrastructure) into oracle/libmac_oracle.so.

Plain gcc, -O2, OpenMP, no fast-math.  Run as ``python -m oracle.build``.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mac_oracle.c")
LIB = os.path.join(HERE, "libmac_oracle.so")


def build(verbose: bool = False, src: str = SRC, out: str = LIB) -> str:
    """Compile `src` (the oracle, or a test's mutated copy of it) into `out`."""
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter",
           src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
