"""include/sanala.h as a C11 header: tests/c_consumer.c (plain C, no C++ and no PyTorch) compiles with
gcc -Wall -Wextra -Werror against it, links every entry point it calls from libsanala.so, and gets each
argument error's status code back on the host (fake device addresses, rejected before any HIP call)."""
import os
import shutil
import subprocess

import pytest

import linear_attention_diffusion_qk_amd as sanala

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INC = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.isdir(ROCM_INC), reason="needs gcc and the ROCm headers")
def test_c_consumer_compiles_links_and_gets_status_codes(tmp_path):
    lib = sanala.load_library()
    libdir = os.path.dirname(lib._name)
    exe = str(tmp_path / "c_consumer")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INC}",
           f"-I{os.path.join(ROOT, 'include')}", os.path.join(ROOT, "tests", "c_consumer.c"), f"-L{libdir}", "-lsanala",
           f"-Wl,-rpath,{libdir}", "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    assert "all checks passed" in run.stdout
