"""Build the CPU oracle (``oracle/liboracle.so``) with the host C compiler.

TEST INFRASTRUCTURE: the oracle is the checker, not the product.  It is
compiled without fast-math and without floating-point contraction so that
every float addition is one IEEE single-precision round-to-nearest-even add.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-std=c99", "-O2", "-fPIC", "-shared", "-fno-fast-math",
          "-ffp-contract=off", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it; return the path."""
    cc = os.environ.get("CC", "gcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc] + CFLAGS + [SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
