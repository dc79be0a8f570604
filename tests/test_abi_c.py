"""The C ABI from plain C: tests/native/abi_c_check.c is compiled as C11 by gcc against
include/pagedkv.h, linked to the built libpagedkv.so and run. It checks that the header is valid
C and exercises the entry points that touch no GPU (pool sizing against the pages' per-token
figure, status strings, the host block manager). No GPU is used."""
import os
import shutil
import subprocess

import pytest

import paged_kv_cache_452_amd as pkv

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("gcc") is None or
                    not os.path.exists(os.path.join(ROCM_INCLUDE, "hip", "hip_runtime_api.h")),
                    reason="needs gcc and the HIP runtime headers")
def test_c_program_uses_the_abi(tmp_path):
    pkv.load_library()  # builds the library when there is none
    libdir = os.path.dirname(pkv.LIB_PATH)
    exe = str(tmp_path / "abi_c_check")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror=implicit-function-declaration",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", ROCM_INCLUDE,
           os.path.join(HERE, "native", "abi_c_check.c"), "-L", libdir, "-lpagedkv",
           f"-Wl,-rpath,{libdir}", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "failures 0" in run.stdout
