"""The tiled quant-pack kernel replaces the division r / S by a table
reciprocal and one exact-remainder refinement step.  This CPU brute force
(tests/division_check.c, built with gcc) checks, on two million residuals of
several kinds, that the refined quotient equals the correctly rounded fp32(r / S)
bit for bit (hence the same rint code), including exact and near half-integer
quotients where a wrong rounding would show."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_reciprocal_refinement_matches_division():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "division_check")
        subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", os.path.join(HERE, "division_check.c"),
                        "-o", exe, "-lm"], check=True)
        out = subprocess.run([exe, "2000000"], capture_output=True, text=True, timeout=120)
    print(out.stdout)
    assert out.returncode == 0, out.stdout + out.stderr
    fields = dict(zip(out.stdout.split()[0::2], map(int, out.stdout.split()[1::2])))
    assert fields["samples"] == 2000000 and fields["exact-half-integer"] > 10000
    assert fields["quotient-differs"] == 0 and fields["code-mismatch"] == 0
