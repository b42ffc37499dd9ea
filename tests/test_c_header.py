"""include/flashnorm.h as a plain C header: a C program (tests/c/abi_from_c.c)
compiled with gcc in C mode, linked against the built libflashnorm.so, runs
the validation paths (no GPU needed: every call is rejected before any HIP
call) and checks statuses, error text and the packed size."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "rmsnorm_projection_gemm_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_header_compiles_as_c_and_validation_works_from_c(tmp_path):
    lib = os.path.join(PKG, "libflashnorm.so")
    if not os.path.exists(lib):
        pytest.skip("libflashnorm.so is not built")
    exe = str(tmp_path / "abi_from_c")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-L", PKG, "-lflashnorm",
           f"-Wl,-rpath,{PKG}", "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr + run.stdout
    assert run.stdout.strip() == "ok"
