"""Mutation check of the oracle's pins, on the CPU.

Each case plants one plausible mistake in a copy of the oracle's C source --
a fold that starts one rank late or runs the other way, a dropped term, the
wrong bfloat16 rounding, the average rounded differently, tree children
folded in the other order or a node's own value folded last, the wrong
segment gathered, segments of floor(N/R), saturating int32 sums, max/min
keeping the older of equal values -- rebuilds that copy in a temporary
directory, and runs the pin suite (tests/test_oracle_pins.py) against it.
Every mistake must make at least one pin fail; the unmutated copy must pass.
The oracle in the repository is never touched.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, text in oracle.c -- present exactly once, replacement)
MUTANTS = [
    ("fold starts one rank late",
     "int c = mod(q - (s + 2) * m, R);",
     "int c = mod(q - (s + 1) * m, R);"),
    ("reduce phase takes the successor's partial",
     "int c = mod(q - (s + 2) * m, R);\n            int p = mod(q - m, R);",
     "int c = mod(q - (s + 2) * m, R);\n            int p = mod(q + m, R);"),
    ("owner's own input dropped",
     "acc_t v = acc_op(dtype, op, in, widen(dtype, send, (size_t)q * N + e));",
     "acc_t v = (s == R - 2) ? in : acc_op(dtype, op, in, widen(dtype, send, (size_t)q * N + e));"),
    ("bfloat16 ties round up instead of to even",
     "if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u) != 0u))",
     "if (lo >= 0x8000u)"),
    ("average multiplies by a rounded reciprocal",
     "a.f = a.f / (float)R;",
     "a.f = a.f * (1.0f / (float)R);"),
    ("tree children folded in descending rank order",
     "for (int ch = 0; ch < R; ++ch)\n        if (parent[ch] == v)",
     "for (int ch = R - 1; ch >= 0; --ch)\n        if (parent[ch] == v)"),
    ("tree node's own value folded last",
     "    acc_t p = widen(dtype, send, (size_t)v * N + e);\n"
     "    for (int ch = 0; ch < R; ++ch)\n"
     "        if (parent[ch] == v)\n"
     "            p = acc_op(dtype, op, p, tree_fold(R, parent, dtype, op, send, N, ch, e));\n"
     "    return p;",
     "    acc_t p = widen(dtype, send, (size_t)v * N + e);\n"
     "    int first = 1;\n"
     "    for (int ch = 0; ch < R; ++ch)\n"
     "        if (parent[ch] == v) {\n"
     "            acc_t t = tree_fold(R, parent, dtype, op, send, N, ch, e);\n"
     "            p = first ? t : acc_op(dtype, op, p, t);\n"
     "            first = 0;\n"
     "        }\n"
     "    if (!first)\n"
     "        p = acc_op(dtype, op, p, widen(dtype, send, (size_t)v * N + e));\n"
     "    return p;"),
    ("gather copies the wrong segment",
     "int c = mod(q - (1 + s) * m, R);",
     "int c = mod(q - s * m, R);"),
    ("segments of floor(N/R) elements",
     "size_t S = (N + (size_t)R - 1) / (size_t)R;\n    size_t b = (size_t)c * S;",
     "size_t S = N / (size_t)R;\n    size_t b = (size_t)c * S;"),
    ("int32 sums saturate instead of wrapping",
     "        r.u = a.u + b.u;",
     "    {\n"
     "        int64_t t = (int64_t)(int32_t)a.u + (int64_t)(int32_t)b.u;\n"
     "        r.u = (uint32_t)(int32_t)(t > 2147483647 ? 2147483647 : t < -2147483647 - 1 ? -2147483647 - 1 : t);\n"
     "    }"),
    ("max/min keep the older of equal values",
     "a_wins = op == ORC_MAX ? a.f > b.f : a.f < b.f;",
     "a_wins = op == ORC_MAX ? a.f >= b.f : a.f <= b.f;"),
]


def _tree_with(tmp, mutation):
    """A copy of what the pins need -- the oracle package, the pin tests, the
    conftest and the golden fixtures -- with `mutation` applied."""
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(tmp, "oracle"),
                    ignore=shutil.ignore_patterns("*.so", "*.tmp*", "__pycache__"))
    os.makedirs(os.path.join(tmp, "tests"))
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(tmp, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(tmp, "tests", "golden"))
    if mutation:
        src = os.path.join(tmp, "oracle", "oracle.c")
        text = open(src).read()
        old, new = mutation
        assert text.count(old) == 1, "mutation anchor not found once: %r" % old[:60]
        open(src, "w").write(text.replace(old, new))


def _run_pins(tmp):
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q",
                           "-p", "no:cacheprovider"],
                          cwd=tmp, env=env, capture_output=True, text=True, timeout=600)


def test_unmutated_copy_passes_the_pins(tmp_path):
    _tree_with(str(tmp_path), None)
    r = _run_pins(str(tmp_path))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_every_planted_mistake_fails_a_pin(tmp_path, name, old, new):
    _tree_with(str(tmp_path), (old, new))
    r = _run_pins(str(tmp_path))
    # pytest exits 1 when tests ran and some failed (a build error would be
    # another code, or a failure of every test: not what is asked here)
    assert r.returncode == 1 and " failed" in r.stdout, (name, r.stdout[-2000:], r.stderr[-1500:])
