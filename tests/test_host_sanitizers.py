"""The library's host code (weight packer, code packer, unpacker, layout
query, offline transforms) built with AddressSanitizer and
UndefinedBehaviorSanitizer and run over round trips and error paths
(tests/cpu/host_sanitize.cpp).  CPU only: no HIP source is compiled here."""

import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "w4a8_quantized_gemm_qoq_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_under_address_and_undefined_behaviour_sanitizers():
    srcs = [os.path.join(CSRC, f) for f in ("status.cpp", "pack.cpp", "transforms.cpp")]
    srcs.append(os.path.join(HERE, "cpu", "host_sanitize.cpp"))
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "host_sanitize")
        cmd = ["g++", "-O1", "-g", "-std=c++17", "-pthread", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", exe]
        subprocess.run(cmd, check=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    print(res.stdout)
    print(res.stderr)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "host_sanitize: ok" in res.stdout
    assert "runtime error" not in res.stderr
