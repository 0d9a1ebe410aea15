"""The C ABI's host-side validation under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/c/abi_validate.c drives every entry point with malformed and well-formed arguments. It is
linked against the ABI's own source (api.cpp, compiled here for the host with g++ and both
sanitizers) and launcher stand-ins (tests/c/launch_stubs.cpp), so no GPU and no kernel is
involved: a malformed call must return its status without reaching a launcher, a well-formed one
must reach exactly one, and the sanitizers abort on any out-of-bounds access, use of freed memory
or undefined behaviour in the host code.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
INC = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}"]


def test_abi_validation_under_sanitizers(tmp_path):
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    if gxx is None or gcc is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("no host compiler or HIP headers")
    objs = []
    for src, cc, std in ((os.path.join(ROOT, "rank_recurrent_state_amd", "csrc", "api.cpp"), gxx, "-std=c++17"),
                         (os.path.join(ROOT, "tests", "c", "launch_stubs.cpp"), gxx, "-std=c++17"),
                         (os.path.join(ROOT, "tests", "c", "abi_validate.c"), gcc, "-std=c11")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        res = subprocess.run([cc, std, "-Wall", "-Werror", *SAN, *INC, "-c", src, "-o", obj],
                             capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
        objs.append(obj)
    exe = str(tmp_path / "abi_validate")
    res = subprocess.run([gxx, *SAN, *objs, "-o", exe, "-L/opt/rocm/lib", "-lamdhip64",
                          "-Wl,-rpath,/opt/rocm/lib", "-lm"], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "abi_validate ok" in res.stdout
