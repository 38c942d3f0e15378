"""The library's host code (quantisers, layouts, sizes, validation) built with
AddressSanitizer (ROCm's clang++ -fsanitize=address for the host: the file has
no device code; g++ lacks the _Float16 type it uses) and run
over every format and layout, the threaded quantiser and every error path
(tests/asan/host_driver.cpp).  Any out-of-bounds access, use after free or leak
aborts the driver."""

import os
import shutil
import subprocess

import pytest

from conftest import ROOT

HERE = os.path.dirname(os.path.abspath(__file__))


CLANG = next((c for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")) if c and os.path.exists(c)), None)


@pytest.mark.skipif(CLANG is None, reason="needs clang++")
def test_host_code_under_address_sanitizer(tmp_path):
    exe = str(tmp_path / "host_asan")
    src = os.path.join(ROOT, "bit_block_scaled_router_amd", "csrc", "w4moe_host.cpp")
    cmd = [CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-pthread",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "bit_block_scaled_router_amd", "csrc"),
           os.path.join(HERE, "asan", "host_driver.cpp"), src, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "ok" in r.stdout
