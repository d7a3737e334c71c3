"""The quantizers' quotient: one correctly rounded reciprocal per row and two
FMAs per element give the correctly rounded FP32 quotient x / s for every FP16
x and every positive FP16 s (checked exhaustively by a small C++ program,
built and run here on the host)."""

import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_reciprocal_fma_quotient_equals_ieee_division():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "quotient_check")
        subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-pthread",
                        os.path.join(HERE, "cpu", "quotient_check.cpp"), "-o", exe], check=True)
        res = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(res.stdout)
    assert res.returncode == 0, res.stdout
    assert "pairs 2015299584 mismatches 0" in res.stdout
