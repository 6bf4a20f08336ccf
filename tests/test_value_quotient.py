"""Host pin of the store kernels' value quotient: rint((v - z) / s) from the
product with the rounded reciprocal plus one fused-multiply-add correction
equals rint of the IEEE quotient for every fp16 scale around every
half-integer (tests/value_quotient.c, compiled with the host C compiler).
The GPU parity tests compare the resulting value codes with the oracle bit
for bit; this test covers the ties (inputs whose quotient is exactly a
half-integer are common with bf16 values and fp16 scales) exhaustively."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_corrected_quotient_rounds_like_the_ieee_quotient(tmp_path):
    exe = str(tmp_path / "value_quotient")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, os.path.join(HERE, "value_quotient.c"), "-lm"],
                   check=True)
    r = subprocess.run([exe, "40"], capture_output=True, text=True, timeout=120)
    print(r.stdout.strip())
    assert r.returncode == 0, r.stdout
    assert "rounding mismatches 0 quotient mismatches 0" in r.stdout
