"""Build libar.so (HIP kernels for gfx950 + host communicator) in-tree.

hipcc cross-compiles for gfx950 without a GPU.  Flags:
  -O3, no fast-math, -ffp-contract=off: every float add is one IEEE add;
  -fno-gpu-flush-denormals-to-zero: denormals are kept, like the host;
  -Xclang -target-feature -Xclang -packed-fp32-ops: no packed fp32 ops
  (the host pass warns that it does not know the feature; harmless).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libar.so")
SOURCES = ["ar_comm.cpp", "ar_ring.hip", "ar_fused.hip", "ar_pipe.hip", "ar_ring_ll.hip", "ar_tree.hip",
           "ar_tree_fused.hip", "ar_util.hip", "ar_noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fno-fast-math", "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile libar.so (to `out`); `defines` are extra -D settings such as
    AR_BLOCK / AR_UNROLL for tuning builds."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ([HIPCC] + FLAGS + ["-D" + d for d in defines]
           + ["-I", os.path.join(ROOT, "include"), "-I", CSRC] + srcs + ["-o", tmp])
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    log = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        sys.stderr.write(log + "\n")
        raise RuntimeError("hipcc failed building libar.so")
    if verbose and log.strip():
        print(log)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
