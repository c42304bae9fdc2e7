"""Builds the C oracle (oracle/ibp_oracle.c) into oracle/liboracle.so.

TEST INFRASTRUCTURE ONLY.  Plain gcc with OpenMP over rows; no intrinsics.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ibp_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose=False, src=SRC, out=LIB, werror=True):
    """Compiles `src` (default: the oracle) into the shared library `out`."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra"]
    if werror:
        cmd.append("-Werror")
    cmd += [src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
