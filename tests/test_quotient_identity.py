"""The KV-cache write divides by k_scale / v_scale with an FMA-corrected
reciprocal product instead of a division instruction.  This CPU test checks,
on random float32 bit patterns and near-integer quotients for scales across
[2^-100, 2^100], that the identity and the range guard it uses give exactly
the IEEE float32 quotient (the oracle's definition of the write)."""
import os
import platform
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(platform.machine() not in ("x86_64", "AMD64"), reason="needs an x86-64 host with FMA")
def test_fma_corrected_quotient_equals_ieee_division(tmp_path):
    exe = tmp_path / "quotient_identity"
    subprocess.check_call(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-std=c11",
                           os.path.join(HERE, "quotient_identity.c"), "-o", str(exe), "-lm"])
    r = subprocess.run([str(exe), "400000"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout
