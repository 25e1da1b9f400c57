"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

oracle.c is compiled with gcc -fsanitize=address,undefined into a temporary library,
and every pin runs against it in a child Python process with the sanitizer runtimes
preloaded: an out-of-bounds access, a use after free or undefined behaviour in the
oracle aborts the child.  A copy with a planted one-past-the-end read must abort, which
shows the sanitizers are live in that process.  No GPU code is built here.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {here!r}]
import oracle, pins
with oracle.using({lib!r}):
    for p in pins.ALL_PINS:
        p()
print("pins-ok", len(pins.ALL_PINS))
"""


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def _build(src_dir, out):
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", os.path.join(src_dir, "oracle.c"), "-o", out, "-lm"],
                   check=True)


def _run_pins(lib):
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join(p for p in (_runtime("libasan.so"), _runtime("libubsan.so")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    code = CHILD.format(root=ROOT, here=HERE, lib=lib)
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=600)


@pytest.fixture(scope="module")
def sanitizers():
    if not (_runtime("libasan.so") and _runtime("libubsan.so")):
        pytest.skip("gcc's sanitizer runtimes are not installed")


def test_pins_under_sanitizers(sanitizers, tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    _build(os.path.dirname(oracle.SRC_PATH), lib)
    r = _run_pins(lib)
    assert r.returncode == 0 and "pins-ok" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]


def test_sanitizers_are_live(sanitizers, tmp_path):
    """A read one past the end of the weight array in the draw must abort the child."""
    d = tmp_path / "planted"
    d.mkdir()
    src_dir = os.path.dirname(oracle.SRC_PATH)
    shutil.copy(os.path.join(src_dir, "oracle.h"), d / "oracle.h")
    src = open(oracle.SRC_PATH).read()
    old = "    for (int64_t v = 0; v < V; ++v)\n        W += w[v];\n    double t = u * W;"
    assert src.count(old) == 1
    (d / "oracle.c").write_text(src.replace(old, old.replace("v < V", "v <= V")))
    lib = str(d / "liboracle_san.so")
    _build(str(d), lib)
    r = _run_pins(lib)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, (r.returncode, r.stderr[-2000:])
