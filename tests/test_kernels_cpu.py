"""Static checks of the gfx950 kernels, compiled on the host (no GPU): no
kernel may keep per-thread arrays in scratch memory or spill registers.  A
kernel that does runs every slot access through private memory, orders of
magnitude slower than its register form (a tuning build with 16 slots per
thread did exactly that)."""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from collective_communication_ring_amd import build

DEVICE_SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]


def _kernel_metadata(src, outdir):
    out = os.path.join(outdir, os.path.basename(src) + ".s")
    flags = [f for f in build.FLAGS if f not in ("-fPIC", "-shared")]
    cmd = ([build.HIPCC] + flags + ["--cuda-device-only", "-S",
                                    "-I", os.path.join(build.ROOT, "include"), "-I", build.CSRC,
                                    os.path.join(build.CSRC, src), "-o", out])
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    text = open(out).read()
    kernels = {}
    for block in re.split(r"\n\s+- \.agpr_count:", text)[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name:
            continue
        fields = {k: int(v) for k, v in re.findall(
            r"\.(private_segment_fixed_size|vgpr_spill_count|sgpr_count|vgpr_count):\s+(\d+)", block)}
        kernels[name.group(1)] = fields
    return kernels


@pytest.mark.skipif(not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None,
                    reason="hipcc is not installed")
def test_no_kernel_uses_scratch_or_spills():
    with tempfile.TemporaryDirectory() as d:
        with ThreadPoolExecutor(max_workers=len(DEVICE_SOURCES)) as ex:
            results = list(ex.map(lambda s: _kernel_metadata(s, d), DEVICE_SOURCES))
    kernels = {}
    for r in results:
        kernels.update(r)
    assert len(kernels) >= 60, sorted(kernels)  # every instantiation was seen
    bad = {k: v for k, v in kernels.items()
           if v.get("private_segment_fixed_size", 0) or v.get("vgpr_spill_count", 0)}
    assert not bad, bad
