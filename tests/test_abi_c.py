"""The C ABI used from plain C: tests/c/abi_smoke.c is compiled as C99 against include/awq.h,
linked against libawq.so and run (it makes no HIP call, so no GPU is needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "post_weight_quantization_channel_amd")
ROCM_INC = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_links_and_calls_the_abi(tmp_path):
    lib = os.path.join(PKG, "libawq.so")
    if not os.path.exists(lib):
        pytest.fail("libawq.so is missing: build it first")
    exe = tmp_path / "abi_smoke"
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", ROCM_INC,
           os.path.join(ROOT, "tests", "c", "abi_smoke.c"), "-o", str(exe),
           "-L", PKG, "-lawq", f"-Wl,-rpath,{PKG}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "C ABI ok" in r.stdout
