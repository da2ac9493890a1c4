"""The float8 encode kernels' quotient method, checked on the CPU.

The kernels replace the IEEE fp32 division x / scale by a reciprocal with one
FMA correction (Markstein's method) for scales in [2^-80, 2^80].  This test
compiles a C restatement of that sequence (tests/native/quotient_check.c)
and compares it with IEEE division for every finite bf16 x, at every 16th
dynamic scale amax/FMAX and at edge scales, for E4M3 (FMAX 448) and E5M2
(FMAX 57344): the codes must agree everywhere.  The clamp-free form used
with dynamic scales is checked over every |x| <= amax of each scale.
The GPU tests then check the kernel itself against the oracle, bit for bit.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_reciprocal_fma_quotient_matches_ieee_division(tmp_path, fmt):
    exe = tmp_path / "quotient_check"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "native", "quotient_check.c"), "-lm"], check=True)
    r = subprocess.run([str(exe), "16", fmt], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
