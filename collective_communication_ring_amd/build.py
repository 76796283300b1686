"""Build libar.so (HIP kernels for gfx950 + host communicator) in-tree.

hipcc cross-compiles for gfx950 without a GPU.  Flags:
  -O3, no fast-math, -ffp-contract=off: every float add is one IEEE add;
  -fno-gpu-flush-denormals-to-zero: denormals are kept, like the host;
  -Xclang -target-feature -Xclang -packed-fp32-ops: no packed fp32 ops
  (the host pass warns that it does not know the feature; harmless).
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

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


def _run(cmd, verbose, what):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    log = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        sys.stderr.write(log + "\n")
        raise RuntimeError("hipcc failed building %s" % what)
    if verbose and log.strip():
        print(log)


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile libar.so (to `out`); `defines` are extra -D settings such as
    AR_BLOCK / AR_UNROLL for tuning builds.  Each source compiles to an
    object on its own (several at once), then one link makes the library."""
    compile_flags = [f for f in FLAGS if f != "-shared"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objdir = tempfile.mkdtemp(prefix="libar_obj_")
    try:
        objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[HIPCC] + compile_flags + ["-D" + d for d in defines] + inc
                + ["-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
        jobs = max(1, min(len(cmds), os.cpu_count() or 1, 8))
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(lambda c: _run(c, verbose, os.path.basename(c[-3])), cmds))
        tmp = out + ".tmp%d" % os.getpid()
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose,
             "libar.so")
        os.replace(tmp, out)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
