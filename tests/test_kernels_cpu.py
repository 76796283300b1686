"""Static checks of the gfx950 kernels, compiled on the host (no GPU).

1. No kernel may keep per-thread arrays in scratch memory or spill registers.
   A kernel that does runs every slot access through private memory, orders
   of magnitude slower than its register form (a tuning build with 16 slots
   per thread did exactly that).
2. In the LL kernels (double binary tree, ring + LL) no vector-memory wait may
   sit between two stores with no load between them.  gfx9 counts loads and
   stores in one in-order counter, so such a wait makes the second store wait
   until the first has reached memory: a round trip per forwarded line, about
   1 us a hop when it happened (from byte-wide table reads and conditional
   loads, which the compiler's wait insertion cannot count)."""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from collective_communication_ring_amd import build

DEVICE_SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]

pytestmark = pytest.mark.skipif(not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc is not installed")


def _compile(src, outdir):
    out = os.path.join(outdir, os.path.basename(src) + ".s")
    flags = [f for f in build.FLAGS if f not in ("-fPIC", "-shared")]
    cmd = ([build.HIPCC] + flags + ["--cuda-device-only", "-S",
                                    "-I", os.path.join(build.ROOT, "include"), "-I", build.CSRC,
                                    os.path.join(build.CSRC, src), "-o", out])
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    return open(out).read()


@pytest.fixture(scope="module")
def assembly():
    """gfx950 assembly of every device source, keyed by file name."""
    with tempfile.TemporaryDirectory() as d:
        with ThreadPoolExecutor(max_workers=len(DEVICE_SOURCES)) as ex:
            texts = list(ex.map(lambda s: _compile(s, d), DEVICE_SOURCES))
    return dict(zip(DEVICE_SOURCES, texts))


def _kernel_metadata(text):
    kernels = {}
    for block in re.split(r"\n\s+- \.agpr_count:", text)[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name:
            continue
        fields = {k: int(v) for k, v in re.findall(
            r"\.(private_segment_fixed_size|vgpr_spill_count|sgpr_count|vgpr_count):\s+(\d+)", block)}
        kernels[name.group(1)] = fields
    return kernels


def _kernel_bodies(text):
    """Instruction text of every kernel, from its label to its first s_endpgm."""
    out = {}
    for m in re.finditer(r"^(_Z\S+):\s*;", text, re.M):
        end = text.find("s_endpgm", m.end())
        out[m.group(1)] = text[m.end():end]
    return out


def _waits_between_stores(body):
    """Vector-memory waits that follow a store and precede the next store with
    no load or atomic in between (in the order the code is laid out)."""
    bad, state = 0, None
    for line in body.split("\n"):
        ins = line.strip()
        if re.match(r"(global|buffer|flat)_(load|atomic)", ins):
            state = "load"
        elif re.match(r"(global|buffer|flat)_store", ins):
            if state == "store-wait":
                bad += 1
            state = "store"
        elif re.match(r"s_waitcnt\s+vmcnt", ins) and state == "store":
            state = "store-wait"
    return bad


def test_no_kernel_uses_scratch_or_spills(assembly):
    kernels = {}
    for text in assembly.values():
        kernels.update(_kernel_metadata(text))
    assert len(kernels) >= 60, sorted(kernels)  # every instantiation was seen
    bad = {k: v for k, v in kernels.items()
           if v.get("private_segment_fixed_size", 0) or v.get("vgpr_spill_count", 0)}
    assert not bad, bad


def test_ll_kernels_issue_stores_back_to_back(assembly):
    seen, bad = 0, {}
    for src in ("ar_tree.hip", "ar_ring_ll.hip"):
        for name, body in _kernel_bodies(assembly[src]).items():
            if "k_tree_ll" not in name and "k_ring_ll" not in name:
                continue
            seen += 1
            n = _waits_between_stores(body)
            if n:
                bad[name] = n
    # one instantiation per dtype, operator (no int32 average) and lines per
    # thread (1 or 4): 22 tree, 22 each for the LL all-reduce and
    # reduce-scatter, 6 LL all-gather
    assert seen == 72, seen
    assert not bad, bad


def test_wait_rule_catches_a_wait_between_stores():
    """The rule itself, on hand-written instruction sequences."""
    ok = ("global_store_dwordx2 v[4:5], v[20:21], off sc1\n"
          "global_store_dwordx2 v[6:7], v[8:9], off sc1\n"
          "global_load_dwordx2 v[10:11], v[12:13], off sc1\n"
          "s_waitcnt vmcnt(0)\n"
          "global_store_dword v[4:5], v14, off\n")
    bad = ("global_store_dwordx2 v[4:5], v[20:21], off sc1\n"
           "s_waitcnt vmcnt(0)\n"
           "v_mov_b32_e32 v20, v13\n"
           "global_store_dwordx2 v[4:5], v[20:21], off sc1\n")
    assert _waits_between_stores(ok) == 0
    assert _waits_between_stores(bad) == 1
