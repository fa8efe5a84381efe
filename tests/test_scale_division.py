"""The quantize kernel forms the group scale RN((max - min) / L) as
q0 = RN(x * RN(1/L)) plus one FMA residual correction.  This checks that it
equals the IEEE quotient for L = 3, 15 and 255: on every 97th positive finite
float and both ends of every binade by default, on all 2^31 - 2^23 of them
with KIVI_EXHAUSTIVE=1 (about 40 s per L)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_fma_corrected_scale_equals_ieee_division(tmp_path):
    exe = str(tmp_path / "scale_division_check")
    subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
                    os.path.join(HERE, "scale_division_check.c"), "-o", exe, "-lm"], check=True)
    stride = "1" if os.environ.get("KIVI_EXHAUSTIVE") else "97"
    r = subprocess.run([exe, stride], capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-2000:]
    assert "mismatches 0" in r.stdout
