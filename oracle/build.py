"""Build the CPU oracle (``oracle/liboracle.so``) with the host C compiler.

TEST INFRASTRUCTURE: the oracle is the checker, not the product.  It is
compiled without fast-math and without floating-point contraction so that
every float addition is one IEEE single-precision round-to-nearest-even add.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")          # one thread
LIB_OMP = os.path.join(HERE, "liboracle_omp.so")  # OpenMP: parallel within a step

CFLAGS = ["-std=c99", "-O2", "-fPIC", "-shared", "-fno-fast-math",
          "-ffp-contract=off", "-Wall", "-Wextra"]


def _compile(out, extra, verbose):
    cc = os.environ.get("CC", "gcc")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [cc] + CFLAGS + extra + [SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile oracle.c twice next to it: liboracle.so (single-threaded) and
    liboracle_omp.so (the same code with its OpenMP loops on).  Returns the
    single-threaded library's path."""
    _compile(LIB_OMP, ["-fopenmp"], verbose)
    return _compile(LIB, ["-Wno-unknown-pragmas"], verbose)


if __name__ == "__main__":
    print(build(verbose=True))
