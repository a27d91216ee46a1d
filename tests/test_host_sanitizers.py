"""The C ABI's host code under AddressSanitizer and UBSan (CPU only).

csrc/api.hip holds no device code: it is copied to a .cpp file and built
with g++ -fsanitize=address,undefined together with stand-in kernel
launchers (tests/host_sanitize/stub_launch.cpp) and a driver
(tests/host_sanitize/driver.cpp) that sends every entry point NULL,
misaligned and out-of-range arguments and a seeded sweep of descriptors.
Any out-of-bounds access, leak or undefined behaviour aborts the driver."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_08_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_sanitize")
HIP_INC = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INC),
                    reason="needs g++ and the HIP headers")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    src = (open(os.path.join(CSRC, "api.hip")).read()
           .replace('#include "../../include/sparse_attn.h"', '#include "sparse_attn.h"'))
    (tmp_path / "api.cpp").write_text(src)
    for f in ("launch.h",):
        shutil.copy(os.path.join(CSRC, f), tmp_path / f)
    shutil.copy(os.path.join(ROOT, "include", "sparse_attn.h"), tmp_path / "sparse_attn.h")
    exe = tmp_path / "driver"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    cmd = ["g++", "-std=c++17", "-O1", "-g", *san, "-D__HIP_PLATFORM_AMD__", "-I", str(tmp_path),
           "-I", HIP_INC, str(tmp_path / "api.cpp"), os.path.join(HERE, "stub_launch.cpp"),
           os.path.join(HERE, "driver.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "all checks passed" in r.stdout
