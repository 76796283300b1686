"""The C ABI used from C: tests/c_abi/allreduce_demo.c includes only ar.h and
the HIP runtime API and links libar.so directly.  Compiling and linking it
runs on the host; running it needs the GPU."""
import os
import shutil
import subprocess

import pytest

from collective_communication_ring_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "c_abi", "allreduce_demo.c")
ROCM = "/opt/rocm"


def _compile(outdir):
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("gcc or the HIP runtime library is not installed")
    if not os.path.exists(build.LIB):
        build.build()
    exe = os.path.join(outdir, "allreduce_demo")
    libdir = os.path.dirname(build.LIB)
    cmd = [gcc, "-std=c99", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(build.ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-o", exe, libdir + "/libar.so", "-Wl,-rpath," + libdir,
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-3000:]
    return exe


def test_c_program_compiles_and_links_against_the_abi(tmp_path):
    assert os.path.exists(_compile(str(tmp_path)))


@pytest.mark.gpu
def test_c_program_runs(tmp_path):
    exe = _compile(str(tmp_path))
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-3000:]
