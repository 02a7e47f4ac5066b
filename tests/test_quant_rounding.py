"""The GPU quantiser computes each code as rint(fl32((x - min) * r)) with r
the hardware reciprocal of the scale (within one ulp of 1/s), falling back to
the IEEE fp32 quotient within 2^-16 of a rounding boundary, and the scale's
division by 15 as a product with an FMA correction.  This checks, on the CPU
with the same fp32 operations, that both equal the IEEE quotients the oracle
uses -- rint(fl32((x - min) / s)) and fl32((max - min) / 15) -- for every
97th positive fp16 scale (each of the three reciprocals within one ulp), 16
minima and every fp16 value in range, and every 97th fp32 value up to 131072
for the division by 15.  The full enumeration (stride 1, e.g. as six runs
with stride 6 and offsets 0-5: 27,205,198,098 code cases, 2,114,583 of them
through the fallback, and 1,207,959,553 divisions by 15) found no
difference."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_division_free_rounding_equals_ieee_quotient(tmp_path):
    exe = tmp_path / "quant_rounding_check"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", str(exe),
                    os.path.join(HERE, "quant_rounding_check.c"), "-lm"], check=True)
    r = subprocess.run([str(exe), "97"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    words = r.stdout.split()
    checked, scales = int(words[1]), int(words[5])
    assert checked > 150_000_000 and scales > 10_000_000 and "mismatches 0" in r.stdout, r.stdout
