"""A plain C99 program compiles against include/*.h, links libs4kv.so and
gets the documented host-side results (tests/c_abi/host_calls.c). CPU only:
nothing it calls reaches a kernel."""

import os
import shutil
import subprocess

import pytest

from int4_kivi_quantized_amd import s4kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_client_builds_links_and_runs(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lib = s4kv.library_path()
    assert os.path.exists(lib), "build libs4kv.so first"
    exe = tmp_path / "host_calls"
    cmd = [cc, "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi", "host_calls.c"), "-o", str(exe),
           "-L", os.path.dirname(lib), "-l:libs4kv.so", "-Wl,-rpath," + os.path.dirname(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout, r.stderr)
