"""The C-ABI layer (csrc/api.cpp: fail-fast shape validation, argument
checks, dispatch) built for the host alone with g++, its kernel launchers
replaced by stubs (tests/c_abi/sanitize_stubs.cpp), under AddressSanitizer and
UndefinedBehaviorSanitizer with no recovery, and driven through every entry
point by tests/c_abi/sanitize_main.c: valid calls reach their launcher once,
refused calls launch nothing, and no check overflows or reads out of bounds."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "int4_kivi_quantized_amd", "csrc")
HIP_INC = "/opt/rocm/include"


def test_api_layer_under_asan_ubsan(tmp_path):
    cxx, cc = shutil.which("g++"), shutil.which("gcc")
    if cxx is None or cc is None or not os.path.isdir(HIP_INC):
        pytest.skip("needs g++, gcc and the HIP headers")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-g", "-O1"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src, extra in ((os.path.join(CSRC, "api.cpp"), ["-D__HIP_PLATFORM_AMD__", "-I", HIP_INC]),
                       (os.path.join(ROOT, "tests", "c_abi", "sanitize_stubs.cpp"),
                        ["-D__HIP_PLATFORM_AMD__", "-I", HIP_INC])):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([cxx, "-std=c++17", "-Wall", "-Werror", *san, *inc, *extra, "-c", src,
                            "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    main_obj = str(tmp_path / "sanitize_main.o")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", *san, *inc, "-c",
                        os.path.join(ROOT, "tests", "c_abi", "sanitize_main.c"), "-o", main_obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "sanitize_main")
    r = subprocess.run([cxx, *san, main_obj, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout, r.stderr[-3000:])
