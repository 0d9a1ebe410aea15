"""The C ABI from plain C (tests/c/abi_smoke.c): it compiles as C against include/seed.h and
links against libseed.so and the HIP runtime's C API (CPU), and runs a prefill-end compression,
a window of decode steps, a compression and a chunk on the GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "abi_smoke.c")
LIBDIR = os.path.join(ROOT, "rank_recurrent_state_amd")


def _build(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None or not os.path.exists(os.path.join(LIBDIR, "libseed.so")):
        pytest.skip("no C compiler or library not built")
    exe = str(tmp_path / "abi_smoke")
    cmd = [cc, "-std=c11", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{os.path.join(ROOT, 'include')}", SRC, "-o", exe, f"-L{LIBDIR}", "-lseed",
           f"-Wl,-rpath,{LIBDIR}", "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe


def test_c_abi_compiles_and_links(tmp_path):
    _build(tmp_path)


@pytest.mark.gpu
def test_c_abi_runs(tmp_path):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = _build(tmp_path)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "abi_smoke ok" in res.stdout
