"""The per-stream scratch table's lifecycle rules, on the host: growth past any fixed number of
streams, reuse and stream-ordered growth, the last-use event of every call and the wait for it while it
is pending (which orders a new stream behind a reused handle after the old kernels), release, and leases
of one stream never overlapping across host threads.  The table header is compiled with g++ (AddressSanitizer and UBSan on) against a
fake backend that stands in for the HIP runtime."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_diffusion_qk_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_scratch_table_lifecycle(tmp_path):
    exe = tmp_path / "scratch_table_check"
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "scratch_table_check.cpp")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-pthread", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", CSRC, src, "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
